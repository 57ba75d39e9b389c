// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// s_waitcnt with vmcnt = VM (0..63), lgkmcnt = 0, expcnt untouched.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (V#) for raw, untyped loads of [base, base + bytes); base wave-uniform.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xFFFFu;  // stride 0
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000u;  // 32-bit data format, no swizzle
  return r;
}

// Byte address in the workgroup's LDS of a __shared__ location.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)p);
}

// Raw buffer loads into LDS (16 or 4 bytes per lane): lane L's bytes at offset `off` of the
// resource land at LDS address m0addr + 16 L (or 4 L); an offset at or past the resource's size
// reads nothing. Written as inline assembly so that the compiler adds no wait for them before
// later LDS reads (it cannot tell which LDS bytes they write): the caller waits (s_waitcnt
// vmcnt, then a barrier) before the destination is read.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_lds16(u32x4 rs, uint32_t off, uint32_t m0addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0addr), "v"(off), "s"(rs) : "memory", "m0");
}
// The same with the nontemporal (streaming) hint, for data read once.
__device__ __forceinline__ void dma_lds16_nt(u32x4 rs, uint32_t off, uint32_t m0addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(m0addr), "v"(off), "s"(rs) : "memory", "m0");
}
__device__ __forceinline__ void dma_lds4(u32x4 rs, uint32_t off, uint32_t m0addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(m0addr), "v"(off), "s"(rs) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt lgkmcnt(0) only (vector memory left in flight).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8)); }

// Wait until at most `n` vector-memory operations of this wave are outstanding (n clamped to 0..16).
__device__ __forceinline__ void wait_vm_lgkm0_dyn(int n) {
  switch (n <= 0 ? 0 : (n >= 16 ? 16 : n)) {
    case 0: wait_vm_lgkm0<0>(); break;
    case 1: wait_vm_lgkm0<1>(); break;
    case 2: wait_vm_lgkm0<2>(); break;
    case 3: wait_vm_lgkm0<3>(); break;
    case 4: wait_vm_lgkm0<4>(); break;
    case 5: wait_vm_lgkm0<5>(); break;
    case 6: wait_vm_lgkm0<6>(); break;
    case 7: wait_vm_lgkm0<7>(); break;
    case 8: wait_vm_lgkm0<8>(); break;
    case 9: wait_vm_lgkm0<9>(); break;
    case 10: wait_vm_lgkm0<10>(); break;
    case 11: wait_vm_lgkm0<11>(); break;
    case 12: wait_vm_lgkm0<12>(); break;
    case 13: wait_vm_lgkm0<13>(); break;
    case 14: wait_vm_lgkm0<14>(); break;
    case 15: wait_vm_lgkm0<15>(); break;
    default: wait_vm_lgkm0<16>(); break;
  }
}

// Workgroup barrier that also stops the compiler from moving memory accesses across it.
// It does not wait for outstanding memory operations; callers issue the s_waitcnt they need.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane 4r+c supplies
// the address of 4 consecutive 16-bit values (columns 4c..4c+3 of row r of a 4x16 block);
// lane n of the group receives column n of rows 0..3.
__device__ __forceinline__ v4i16 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(const lds_void_t*)p);
}

__device__ __forceinline__ bf16x8 concat_tr(const v4i16& lo, const v4i16& hi) {
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_round(float x) { return (float)(__bf16)x; }

// Cross-lane xor shuffle within a wave (lanes l and l^mask).
__device__ __forceinline__ float xor_shuffle(float v, int mask) {
  int lane = __lane_id();
  int src = lane ^ mask;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

// Reductions over the four lanes {l, l^16, l^32, l^48} with the gfx950 permlane swaps
// (VALU only). permlane32_swap of a register with itself yields, in some order, the
// values of lanes l and l^32; permlane16_swap likewise for l and l^16. Max and sum are
// symmetric, so the order does not matter and all four lanes end with the same result.
// The maximum is IEEE maximum (NaN-propagating, v_maximum3_f32): unlike fmaxf it needs no
// canonicalising moves of the swapped values.
__device__ __forceinline__ float max4_x16_x32(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4_x16_x32(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Map a linear workgroup id so that consecutive logical ids land on the same XCD
// (workgroups are dispatched round-robin over the nx XCDs).
__device__ __forceinline__ int xcd_local_id(int id, int n, int nx = 8) {
  return (nx > 1 && n % nx == 0) ? (id % nx) * (n / nx) + id / nx : id;
}

}  // namespace sa
