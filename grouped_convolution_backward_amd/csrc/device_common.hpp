// Device helpers shared by the HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include "wgrad_internal.hpp"

namespace wgrad {
namespace dev {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int V> struct VecT;
template <> struct VecT<8> { typedef u32x4 T; };
template <> struct VecT<4> { typedef u32x2 T; };
template <> struct VecT<2> { typedef uint32_t T; };
template <> struct VecT<1> { typedef uint16_t T; };

__device__ __forceinline__ uint32_t magic_div(uint32_t n, MagicU32 m) {
    return (__umulhi(m.mul, n) + n) >> m.shift;
}

// fp32 -> bf16, round to nearest even, in hardware (v_cvt_pk_bf16_f32; a
// NaN stays a NaN). Against the integer rounding sequence it replaces, this
// took 2.6-2.9 us off the row-ring backward-data kernel, whose stores
// convert every dX element.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ void store_out(void* out, int mode, int64_t e, float v) {
    if (mode == OUT_BF16) {
        static_cast<uint16_t*>(out)[e] = f32_to_bf16(v);
    } else if (mode == OUT_FP16) {
        static_cast<_Float16*>(out)[e] = (_Float16)v;
    } else {
        static_cast<float*>(out)[e] = v;
    }
}

// Workgroups are dispatched to the 8 XCDs round-robin by id. Renumber them so
// that each XCD receives one contiguous range of logical ids: logical
// neighbours (same reduction slice, adjacent tiles or groups) then share an
// L2 instead of being spread over eight.
__device__ __forceinline__ int xcd_logical_id(int hw, int total) {
    const int q = total >> 3, rem = total & 7;
    const int xcd = hw & 7, slot = hw >> 3;
    return xcd * q + min(xcd, rem) + slot;
}

template <bool F16>
__device__ __forceinline__ void mfma_step32(const i16x8& a, const i16x8& b, f32x16& c) {
    if constexpr (F16)
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ void mfma_step16(const i16x8& a, const i16x8& b, f32x4& c) {
    if constexpr (F16)
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Transposed LDS read: within each 16-lane group, lane i supplies the address
// of 4 consecutive 16-bit elements and lane j receives element j%4 of lanes
// j/4, j/4+4, j/4+8, j/4+12. With lane i pointing at row (i%16)/4, column
// (i%4)*4 of a K-outer tile, lane j receives column j of 4 consecutive rows:
// one MFMA operand run along the reduction axis.
__device__ __forceinline__ i16x8 tr_frag(const uint16_t* p, int row_pitch) {
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * row_pitch));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Raw buffer loads: an offset at or past the buffer's size returns zeros in
// hardware, so bounds and padding checks become a select on the offset
// instead of a branch around the load. Buffers are below 2 GiB, so the
// offset kBufOob is always out of range.
constexpr uint32_t kBufOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    // word 3 = 0x00020000: 32-bit data format for untyped loads on gfx9-family parts
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Stores of fp32 split-K partials, which the reduce kernel reads next, into
// one workspace slice (a buffer of at most 2 GiB; e is the element offset in
// it). They are device-scope stores (cache policy SC1): on the dense split-K
// shapes this shortened the time between the end of the main kernel and the
// reduce kernel's work by about 1 us against plain or nontemporal stores,
// consistent with the partials not being left in this XCD's L2 for the
// end-of-kernel writeback. A buffer-store builtin, not inline assembly, so
// that the compiler sees the store and guards its data registers.
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ void store_partial4(__amdgpu_buffer_rsrc_t r, int64_t e, const f32x4& v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)(e * 4), 0, kCpolSc1);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

// Direct buffer-to-LDS load of 16 bytes per lane (gfx950): lane t's bytes land
// at LDS byte address lds + 16*t; an out-of-range offset writes zeros. Issued
// from inline assembly so that the compiler does not place its own
// "wait for every LDS-bound load" before later LDS reads: the callers wait
// with explicit vmcnt counts for exactly the loads they consume. desc is the
// buffer descriptor as four scalar words (see buf_desc).
__device__ __forceinline__ u32x4 buf_desc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 d;
    d[0] = (uint32_t)a;
    d[1] = (uint32_t)(a >> 32) & 0xffffu;   // stride 0
    d[2] = bytes;
    d[3] = 0x00020000u;
    return d;
}
// M0 is listed as clobbered; the compiler reserves it and uses it for nothing
// else in these kernels (checked in their assembly), hence the pragma.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_load16(const u32x4& desc, uint32_t lds_byte, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_byte), "v"(voff), "s"(desc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}

// s_waitcnt immediate that waits until at most N vector-memory operations of
// this wave are outstanding and does not wait on LDS/scalar or export counters
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
constexpr int kWaitVm = (N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8);

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its global stores (__syncthreads also fences global
// memory, which would stall on outstanding stores for a microsecond or more).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Depthwise products: a * b summed over the two 16-bit halves, plus c, in
// fp32 (v_dot2_f32_bf16 / v_dot2_f32_f16). The halves hold one channel at two
// reduction positions, packed by pair_lo / pair_hi.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <bool F16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (F16)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
// (lo half of a, lo half of b) and (hi half of a, hi half of b)
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Instruction-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100,
              kSchedDsWrite = 0x200;

// LDS row pad (elements): 32 elements = 64 bytes, which puts the four rows a
// 16-lane group reads in one transposed read on disjoint bank ranges.
constexpr int kLdsPad = 32;


}  // namespace dev
}  // namespace wgrad
