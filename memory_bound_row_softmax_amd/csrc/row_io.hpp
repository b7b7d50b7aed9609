// row_io.hpp -- a lane's share of a row: which chunks it owns, loads, masks, stores.
//
// A lane owns C chunks of its row (chunk = 16 bytes): chunk i is ln.chunk(i) (a
// Lane).  A whole row on a group of R lanes: lane l owns chunks l + i * R, so for a
// fixed i the R lanes touch R consecutive chunks and each load instruction of a
// wave covers contiguous memory (1 KiB when R >= 64).  A row split over G
// workgroups: see lane_of.  All C loads are issued before any value is used
// and none sits behind a branch (except on the per-element path of unaligned fp32
// rows, whose values need no conversion after the load).
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

#include "configs.hpp"
#include "vec_io.hpp"

namespace rr {

struct RowView {
    Buf buf;
    uint32_t base;     // byte offset of the row inside buf
    uint32_t end = 0;  // byte offset inside buf where the row ends; 0 if not known
                       // (the per-element path then reads and writes element by
                       // element throughout)
};

// Where a lane's chunks lie in its row: chunk i is first + off(i).  The lane's
// chunks come in rounds of q (one granule of a split row, see lane_of): off(i) =
// (i / q) * stride + (i % q) * step.  With q = 1 that is first + i * stride.
struct Lane {
    int first;
    int stride;
    int step = 0;
    int q = 1;
    __device__ __forceinline__ int off(int i) const { return (i / q) * stride + (i % q) * step; }
    __device__ __forceinline__ int chunk(int i) const { return first + off(i); }
};

// The layout of lane l of workgroup `member` of the G workgroups that share a row,
// for kernel family OP (configs.hpp).  G == 1: the whole row, lane l owns chunks l +
// i * R.  G > 1: the row is cut into granules of K chunks (configs.hpp,
// split_granule), member m owns the granules j with j % G == m, and its chunk k = i *
// R + l (granule k / K of its own, place k % K in it) is chunk ((k / K) * G + m) * K
// + k % K of the row.  For each i the R lanes still read R consecutive chunks.  With
// K = C * R each member holds one contiguous part of the row.  With small granules
// the G members get equal shares of any row (to one granule), and for G = 8 each
// XCD's share of every row is one class of 4 KiB granules (address bits 12..14), as
// in the copy that MI355X ran fastest (copy.hip).
template <int OP, class E, int C, int R, int G>
__device__ __forceinline__ Lane lane_of(int member, int l) {
    if constexpr (G == 1) {
        return {l, R};
    } else {
        constexpr int K = split_granule(OP, C, R, G);
        if constexpr (K <= R) {
            static_assert(R % K == 0, "a granule divides the lanes' chunks of one round");
            return {((l / K) * G + member) * K + l % K, R * G};
        } else {
            static_assert(K % R == 0 && C % (K / R) == 0, "a lane's chunks fill whole granules");
            return {member * K + l, G * K, R, K / R};
        }
    }
}

// The inverse of lane_of: the member, lane and register chunk i (of C) whose part
// holds chunk k >= 0 of the row; i >= C when k lies past every lane's part.  The
// divisors are compile-time constants.
template <int OP, class E, int C, int R, int G>
__device__ __forceinline__ void chunk_owner(int k, int &member, int &l, int &i) {
    if constexpr (G == 1) {
        member = 0;
        l = k % R;
        i = k / R;
    } else {
        constexpr int K = split_granule(OP, C, R, G);
        if constexpr (K <= R) {
            // chunk(i) = gi * K + k % K + i * R * G with gi = (l / K) * G + member
            const int rem = k % (R * G), gi = rem / K;
            member = gi % G;
            l = (gi / G) * K + rem % K;
            i = k / (R * G);
        } else {
            // chunk(i) = member * K + (i % q) * R + l + (i / q) * G * K, q = K / R
            const int rem = k % (G * K), in = rem % K;
            member = rem / K;
            l = in % R;
            i = (k / (G * K)) * (K / R) + in / R;
        }
    }
}

// Whether every chunk that member `member` of a row's G workgroups owns (C chunks
// in each of its lanes, layout of lane_of) lies wholly inside a row of N elements:
// whether the last chunk of its last lane does.
template <int OP, class E, int C, int R, int G>
__device__ __forceinline__ bool part_full(int member, int N) {
    return ((int64_t)lane_of<OP, E, C, R, G>(member, R - 1).chunk(C - 1) + 1) * E::VPC <=
           (int64_t)N;
}

// The same for a lane group that holds chunks chunk0 + i * R + l of a row (block
// kernels, one tile of a long row).
template <class E, int C, int R>
__device__ __forceinline__ bool part_full_at(int chunk0, int N) {
    return (int64_t)(chunk0 + C * R) * E::VPC <= (int64_t)N;
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

// The lane's first chunk, as a value the compiler cannot trace back to how it was
// computed.  The predicated stores of the block kernels take their addresses from
// it, so that the addresses of a part are formed where they are used: otherwise the
// compiler keeps the C addresses of the loads live in registers until the stores
// that reuse them (up to 40 more registers a lane).  The persistent kernels keep
// their addresses from row to row anyway, and there the stores go out back to back.
__device__ __forceinline__ int fresh_first(Lane ln) {
    int f = ln.first;
    asm volatile("" : "+v"(f));
    return f;
}

// POLICY: kStreamLoad for data read once, kReuseLoad for data read by every row.
template <class E, int C, int R, bool VEC, int POLICY = kStreamLoad>
__device__ __forceinline__ void load_part(RowView rv, Lane ln, float *v) {
    constexpr int VPC = E::VPC;
    if constexpr (VEC) {
        u32x4 raw[C];
#pragma unroll
        for (int i = 0; i < C; ++i)
            raw[i] = buf_load16<POLICY>(rv.buf, rv.base + (uint32_t)ln.chunk(i) * 16u);
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
            const uint32_t first = (uint32_t)ln.chunk(i) * VPC;
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
            const uint32_t first = (uint32_t)ln.chunk(i) * VPC;
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
            const uint32_t first = (uint32_t)ln.chunk(i) * VPC;
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
__device__ __forceinline__ void load_part_raw(RowView rv, Lane ln, float *v) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const u32x4 raw =
            buf_load16<POLICY>(rv.buf, rv.base + (uint32_t)ln.chunk(i) * 16u);
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
// OPAQUE (persistent kernels, whose row loop keeps the layout and N fixed): the lane's
// count of elements left in the row passes through an empty asm statement, so that
// the comparisons stay inside the row loop, where they run only for a part that is
// not full.  Left to itself, the compiler hoists all P comparisons out of the loop,
// and their P lane masks and element indices stay live in registers for every row
// (116 spilled scalar registers and some 15 vector registers in the 64-value fp32
// stream kernel).
template <class E, int C, int R, bool OPAQUE = false>
__device__ __forceinline__ void mask_part(Lane ln, int N, float fill, float *v) {
    constexpr int VPC = E::VPC;
    int left = N - ln.first * VPC;  // negative or zero: nothing of the row
    if constexpr (OPAQUE) asm volatile("" : "+v"(left));
    // Compared with the lane's count of elements left, so that one register holds
    // what the comparisons need (an element index per chunk would be shared with
    // the loads' addresses and stay live until here).
#pragma unroll
    for (int i = 0; i < C; ++i) {
#pragma unroll
        for (int e = 0; e < VPC; ++e)
            if (ln.off(i) * VPC + e >= left) v[i * VPC + e] = fill;
    }
}

// BOUNDED: the buffer resource holds only this row and ends where it ends, as in the
// persistent kernels; the hardware's range check
// then drops the stores of chunks past it, and whole waves per row store every chunk
// with no predicate.  Left to a per-chunk predicate in a row loop, the compiler hoists
// the chunks' comparisons out of the loop and keeps their lane masks live (spilled
// scalar registers).  Otherwise (block kernels, whose lane groups of fewer than 64
// lanes share one buffer across rows) each chunk is stored only if it lies in the row.
template <class E, int C, int R, bool VEC, bool BOUNDED = false>
__device__ __forceinline__ void store_part(RowView rv, Lane ln, int N, bool valid,
                                           bool full, const float *v) {
    constexpr int VPC = E::VPC;
    if constexpr (VEC) {
        if constexpr (BOUNDED && R >= 64) {
            if (valid) {
#pragma unroll
                for (int i = 0; i < C; ++i)
                    buf_store16(rv.buf, rv.base + (uint32_t)ln.chunk(i) * 16u,
                                encode<E>(v + i * VPC));
            }
        } else {
            const int f = fresh_first(ln);
            const int left = N - ln.first * VPC;  // as in mask_part
#pragma unroll
            for (int i = 0; i < C; ++i) {
                if (valid && (full || ln.off(i) * VPC < left))
                    buf_store16(rv.buf, rv.base + (uint32_t)(f + ln.off(i)) * 16u,
                                encode<E>(v + i * VPC));
            }
        }
    } else {
        // As for the loads: whole chunks inside the row are one 16-byte store, the rest
        // element by element.
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int first = ln.chunk(i) * VPC;
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
