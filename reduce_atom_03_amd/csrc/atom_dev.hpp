// atom_dev.hpp -- device helpers for the gfx950 Atom kernels: 128-bit
// global loads/stores (optionally non-temporal), bf16 widening and
// round-to-nearest-even narrowing, and the agent-coherent ring accesses and
// flag operations used by SNAC.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kargs.hpp"

namespace atom {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- 16-byte memory operations (global_load/store_dwordx4) -------------

__device__ __forceinline__ u32x4 ld16(const void* p)
{
    return *reinterpret_cast<const u32x4*>(p);
}

// Streaming read: each input byte is read exactly once, so the load is
// marked non-temporal to keep it from displacing reusable cache lines.
__device__ __forceinline__ u32x4 ld16_stream(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Buffer resources (gfx9 raw buffers: base, 32-bit range, no stride) and
// the cache-policy operand of buffer loads and stores.
constexpr int kBufRsrcWord3 = 0x00020000;   // gfx9 raw buffer: 32-bit data format
constexpr int kCpolNt = 2;                  // cache-policy operand: nt (streaming)
constexpr int kCpolSc1 = 16;                // cache-policy operand: sc1

// Output store of 16 bytes at base + off, with base wave-uniform (the
// tile's, or the row's, start) and off the lane's offset from it. The store
// goes through a buffer resource so that the cache policy is an immediate
// operand of each branch: written as `nt ? nontemporal store : store`
// through a pointer, the compiler merges the two stores into one ordinary
// store and drops the non-temporal hint, so the streaming policy never
// reaches the hardware (measured on MI355X: an 8-way reduce ran 13 % slower
// with the merged store when the caches held dirty lines).
__device__ __forceinline__ void st16(char* base, uint32_t off, u32x4 v, bool nt)
{
    const auto r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, kBufRsrcWord3);
    if (nt)
        __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0, kCpolNt);
    else
        __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0, 0);
}

// ---- element conversions ----------------------------------------------

// bf16 -> binary32 is exact: the bf16 pattern is the upper half of the
// binary32 pattern. A 32-bit word holds two bf16, element 0 in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Two binary32 -> two bf16 packed in one word (element 0 low), rounded to
// nearest with ties to even by gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2 f = {lo, hi};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x)
{
    return static_cast<uint16_t>(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

// One 16-byte slot of binary32 sums: init from rank 0, add the others in
// rank order, pack with one round-to-nearest-even narrowing.
template <typename T> struct SlotAcc;

template <> struct SlotAcc<uint16_t> {   // 8 bf16 per slot
    float v[8];
    __device__ __forceinline__ void init(u32x4 x)
    {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            v[2 * w] = bf16_lo(x[w]);
            v[2 * w + 1] = bf16_hi(x[w]);
        }
    }
    __device__ __forceinline__ void add(u32x4 x)
    {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            v[2 * w] = v[2 * w] + bf16_lo(x[w]);
            v[2 * w + 1] = v[2 * w + 1] + bf16_hi(x[w]);
        }
    }
    __device__ __forceinline__ u32x4 pack() const
    {
        u32x4 r;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            r[w] = pack_bf16x2(v[2 * w], v[2 * w + 1]);
        return r;
    }
};

template <> struct SlotAcc<float> {      // 4 fp32 per slot
    float v[4];
    __device__ __forceinline__ void init(u32x4 x)
    {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            v[w] = __uint_as_float(x[w]);
    }
    __device__ __forceinline__ void add(u32x4 x)
    {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            v[w] = v[w] + __uint_as_float(x[w]);
    }
    __device__ __forceinline__ u32x4 pack() const
    {
        u32x4 r;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            r[w] = __float_as_uint(v[w]);
        return r;
    }
};

// ---- byte-shifted slots (a source and a destination off each other's
// 16-byte alignment) ------------------------------------------------------
// A lane holds the source vector v (bytes [16v, 16v + 16) of the address
// space) and gets vector v - 1 from its neighbour; the destination slot it
// writes is 16 bytes that straddle the two. funnel16(lo, hi, d): the 16
// bytes that begin 16 - d bytes into the string lo | hi (lo's bytes first),
// d in 0..15 (d = 0 gives hi). d is wave-uniform, so the dword selection is
// a uniform branch and the shifts are v_alignbyte_b32.
__device__ __forceinline__ u32x4 funnel16(u32x4 lo, u32x4 hi, int d)
{
    const int s = 16 - d;                          // 1..16 bytes into lo | hi
    const uint32_t r = static_cast<uint32_t>(s & 3);
    const uint32_t c0 = lo[0], c1 = lo[1], c2 = lo[2], c3 = lo[3];
    const uint32_t c4 = hi[0], c5 = hi[1], c6 = hi[2], c7 = hi[3];
    u32x4 o;
    switch (s >> 2) {
    case 0:
        o = u32x4{__builtin_amdgcn_alignbyte(c1, c0, r), __builtin_amdgcn_alignbyte(c2, c1, r),
                  __builtin_amdgcn_alignbyte(c3, c2, r), __builtin_amdgcn_alignbyte(c4, c3, r)};
        break;
    case 1:
        o = u32x4{__builtin_amdgcn_alignbyte(c2, c1, r), __builtin_amdgcn_alignbyte(c3, c2, r),
                  __builtin_amdgcn_alignbyte(c4, c3, r), __builtin_amdgcn_alignbyte(c5, c4, r)};
        break;
    case 2:
        o = u32x4{__builtin_amdgcn_alignbyte(c3, c2, r), __builtin_amdgcn_alignbyte(c4, c3, r),
                  __builtin_amdgcn_alignbyte(c5, c4, r), __builtin_amdgcn_alignbyte(c6, c5, r)};
        break;
    case 3:
        o = u32x4{__builtin_amdgcn_alignbyte(c4, c3, r), __builtin_amdgcn_alignbyte(c5, c4, r),
                  __builtin_amdgcn_alignbyte(c6, c5, r), __builtin_amdgcn_alignbyte(c7, c6, r)};
        break;
    default:
        o = hi;
        break;
    }
    return o;
}

// The vector of the lane below in the wave; lane 0 gets `carry` (the
// previous row's lane 63, or a vector loaded for it). Every lane of the
// wave must be active.
__device__ __forceinline__ u32x4 from_lane_below(u32x4 v, u32x4 carry)
{
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = static_cast<uint32_t>(__shfl_up(static_cast<int>(v[i]), 1, 64));
    return (threadIdx.x & 63) == 0 ? carry : r;
}

__device__ __forceinline__ u32x4 lane63(u32x4 v)
{
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v[i]), 63));
    return r;
}

// Bytes [p0, p1) of slot `v` to the 16-byte aligned address `slot`, in
// units of es bytes (the element size; p0 and p1 are multiples of it).
__device__ __forceinline__ void store_slot_part(char* slot, u32x4 v, int p0, int p1, int es)
{
    for (int p = p0; p < p1; p += es) {
        const uint32_t w = v[p >> 2];
        if (es == 4)
            *reinterpret_cast<uint32_t*>(slot + p) = w;
        else if (es == 2)
            *reinterpret_cast<uint16_t*>(slot + p) = static_cast<uint16_t>(w >> (8 * (p & 3)));
        else
            *reinterpret_cast<uint8_t*>(slot + p) = static_cast<uint8_t>(w >> (8 * (p & 3)));
    }
}

// ---- XCD-aware tile order ----------------------------------------------
// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on
// XCD b mod 8). Renumbering so that XCD x's workgroups own one contiguous
// eighth of the grid keeps each XCD's address translations and DRAM pages
// local instead of every XCD touching every page. A bijection on [0, nb)
// for any nb; if dispatch were not round-robin it is still a permutation.
constexpr int kXcds = 8;

__device__ __forceinline__ int64_t xcd_slot(int64_t b, int64_t nb)
{
    const int64_t q = nb / kXcds, r = nb % kXcds;
    const int64_t x = b % kXcds, i = b / kXcds;
    return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Tile of the workgroup in grid-stride round `round`.
__device__ __forceinline__ int64_t tile_of(int64_t round_base, bool remap)
{
    const int64_t b = blockIdx.x, nb = gridDim.x;
    return round_base + (remap ? xcd_slot(b, nb) : b);
}

// ---- element access for the element-wise (unaligned) paths ------------

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {   // bf16 storage
    static constexpr int kSize = 2;
    __device__ static float load(const void* base, int64_t i)
    {
        return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
    }
    __device__ static void store(void* base, int64_t i, float v)
    {
        static_cast<uint16_t*>(base)[i] = f32_to_bf16_bits(v);
    }
};
template <> struct Elem<float> {
    static constexpr int kSize = 4;
    __device__ static float load(const void* base, int64_t i) { return static_cast<const float*>(base)[i]; }
    __device__ static void store(void* base, int64_t i, float v) { static_cast<float*>(base)[i] = v; }
};

// ---- SNAC hand-off ------------------------------------------------------
// Staged data written by one workgroup is consumed by workgroups that may
// run on another XCD, each XCD with its own L2. Rather than fence with the
// agent-scope release/acquire (which writes back, then invalidates, a whole
// L2 per task), the staging ring is accessed only with agent-coherent
// 16-byte operations: buffer loads and stores carrying the sc1 cache-policy
// bit. An sc1 store writes through the XCD's L2 and an sc1 load does not
// return a line that an L2 kept from before; these are the cache policies
// the compiler itself gives relaxed agent-scope atomic loads and stores, on
// which the cross-XCD flag polling below already relies. The buffer
// resource covers [base, base + bytes), and the hardware drops accesses
// outside it.

// Bytes rounded up to whole 16-byte vectors.
__device__ __forceinline__ int64_t ceil16(int64_t bytes) { return (bytes + 15) & ~int64_t(15); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ring_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             kBufRsrcWord3);
}

__device__ __forceinline__ u32x4 ld16_agent(__amdgpu_buffer_rsrc_t r, int64_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kCpolSc1);
}

__device__ __forceinline__ void st16_agent(__amdgpu_buffer_rsrc_t r, int64_t off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0, kCpolSc1);
}

// Streaming 16-byte load through a buffer resource: the stream's base stays
// in scalar registers and each lane supplies a 32-bit offset, so a kernel
// reading P streams holds no 64-bit per-lane address per stream in VGPRs
// (the 8-way reduce: 65 -> 50 VGPRs). The resource covers
// [base, base + bytes); the hardware drops accesses outside it.
// Non-temporal, like ld16_stream.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             kBufRsrcWord3);
}

__device__ __forceinline__ u32x4 ld16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kCpolNt);
}

// Waits until every vector memory operation of this wave has completed
// (for sc1 stores: written through to the agent-coherent level).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Kernel arguments sit in memory written just before the launch, and the
// scalar loads that read them form chains (a segment's source pointer is
// read once its index is known, a count once the segment is), each link a
// scalar-cache miss on a fresh launch. One load from each 64-byte line the
// first steps read, all issued before anything waits, fills those lines at
// once, so the chained loads that follow hit. The values are only consumed
// by an empty asm statement. Measured on MI355X (median kernel durations in
// a kernel trace): the staged AllGather and AllReduce of 8 x 8 KiB 8.72 ->
// 8.08 us, the zero-staging AllGather of 8 x 8 KiB 3.44 -> 3.20 us.
__device__ __forceinline__ void touch_arg_lines(const void* p0, const void* p1, const void* p2,
                                                const void* p3, const void* p4, const void* p5,
                                                const void* p6, const void* p7, const void* p8,
                                                const void* p9)
{
    const auto ld = [](const void* p) { return *static_cast<const uint32_t*>(p); };
    asm volatile("" ::"s"(ld(p0)), "s"(ld(p1)), "s"(ld(p2)), "s"(ld(p3)), "s"(ld(p4)), "s"(ld(p5)),
                 "s"(ld(p6)), "s"(ld(p7)), "s"(ld(p8)), "s"(ld(p9)));
}

// The first line of the hidden launch arguments (grid and workgroup sizes).
__device__ __forceinline__ const void* hidden_args()
{
    return (const void*)__builtin_amdgcn_implicitarg_ptr();
}

__device__ __forceinline__ unsigned long long flag_load_relaxed(const unsigned long long* f)
{
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void flag_add_relaxed(unsigned long long* f, unsigned long long v)
{
    __hip_atomic_fetch_add(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace atom
