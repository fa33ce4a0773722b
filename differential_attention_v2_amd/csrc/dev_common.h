// Device-side building blocks shared by the libdiffattn kernels (gfx950 / CDNA4).
//
// Lane layouts used throughout (wave64):
//   v_mfma_f32_32x32x16_bf16  A[m][k]: lane l holds row m = l%32, k = 8*(l/32) + 0..7
//                             B[k][n]: lane l holds col n = l%32, k = 8*(l/32) + 0..7
//                             C[m][n]: lane l, reg i -> m = 8*(i/4) + 4*(l/32) + i%4, n = l%32
//   v_mfma_f32_16x16x32_bf16  A: row l%16, k = 8*(l/16) + 0..7;  B: col l%16, same k
//                             C: lane l, reg i -> m = 4*(l/16) + i, n = l%16
//   ds_read_b64_tr_b16        within each 16-lane group, output lane i element j is
//                             element (i%4) of the 8 bytes addressed by lane 4*j + i/4.
//                             Sixteen lanes that address a row-major 4-row x 16-column
//                             block (lane s -> row s/4, columns 4*(s%4)..+3) therefore
//                             receive lane = column, elements = the 4 rows.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read of 4 bf16 (see layout note above).
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, const_cast<bf16*>(p)));
  return __builtin_bit_cast(bf16x4, t);
}
__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Value held by lane l^32 (the partner in the other half-wave); lo = (lane < 32).
// permlane32_swap(v, v) returns (v[l], v[l+32]) on lanes < 32 and (v[l-32], v[l]) above.
__device__ __forceinline__ float partner32(float v, bool lo) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(lo ? r[1] : r[0]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum of the two bf16 values of a packed pair, accumulated in fp32.
__device__ __forceinline__ float dot2_ones(bf16x2 p, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Direct global -> LDS copy of 16 bytes per lane with a scalar 64-bit base and a
// per-lane 32-bit byte offset (the "saddr" form: no per-lane 64-bit address
// arithmetic): lane l's bytes land at lds_addr + 16*l, lds_addr being the
// wave-uniform LDS byte address of lane 0's 16 bytes.  Issued as inline asm so the
// compiler does not insert conservative vmcnt waits in front of unrelated LDS
// reads; the caller waits on vmcnt before the barrier that publishes the data.
__device__ __forceinline__ void dma16_saddr(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  // one wait state between the M0 write and the copy that reads it
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// vmcnt(0) as a builtin (expcnt/lgkmcnt left at their maxima), visible to the
// compiler's own wait-count tracking: loads issued before it need no later wait.
__device__ __forceinline__ void wait_vmcnt0_builtin() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace diffattn
