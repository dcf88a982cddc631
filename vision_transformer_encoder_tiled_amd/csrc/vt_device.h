// Device-side helpers shared by the gfx950 kernels: bf16 conversion, vector
// types for the MFMA builtins, wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace vt {

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
// fp32 -> fp16 pair, round to nearest even (v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2_t v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
// 3D RoPE on 8 rotation pairs, rotate-half pairing (x_j, x_{j+40} of a head
// of 80), then a scale and fp16 rounding.  a holds x_j .. x_{j+7} and b the
// partners x_{j+40} .. x_{j+47} (bf16), cs[2i], cs[2i+1] = cos, sin of pair
// j+i.  o1 = (a cos - b sin) sc, o2 = (b cos + a sin) sc, every product
// rounded on its own (no contraction into fmas), so that the result does not
// depend on what the compiler knows at the call site: the pack kernel and
// the QKV GEMM epilogue produce the same bits.
__device__ __forceinline__ void rope8_f16(uint4 a, uint4 b, const float (&cs)[16], float sc, uint4* o1,
                                          uint4* o2) {
#pragma clang fp contract(off)
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
  uint32_t r1[4], r2[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float x1l = __uint_as_float(aw[j] << 16), x1h = __uint_as_float(aw[j] & 0xffff0000u);
    const float x2l = __uint_as_float(bw[j] << 16), x2h = __uint_as_float(bw[j] & 0xffff0000u);
    const float cl = cs[4 * j], sl = cs[4 * j + 1], ch = cs[4 * j + 2], sh = cs[4 * j + 3];
    r1[j] = pack_f16x2((x1l * cl - x2l * sl) * sc, (x1h * ch - x2h * sh) * sc);
    r2[j] = pack_f16x2((x2l * cl + x1l * sl) * sc, (x2h * ch + x1h * sh) * sc);
  }
  *o1 = make_uint4(r1[0], r1[1], r1[2], r1[3]);
  *o2 = make_uint4(r2[0], r2[1], r2[2], r2[3]);
}

__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// GELU, tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3),
// evaluated as x * sigmoid(2u) = x / (1 + 2^(-2u log2 e)) with the hardware
// exp2 and reciprocal (about 1 ulp each; the result is rounded to bf16).
// Large negative x: the exponential overflows to +inf and the result is -0.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float c1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float c3 = c1 * 0.044715f;
  const float x2 = x * x;
  const float e = __builtin_amdgcn_exp2f(x * fmaf(c3, x2, c1));
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}
// GELU, exact form with the device erf.
__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.7071067811865476f));
}

// Slot of index k inside its group of 16 when a [.][16 k] operand is fed as
// the k-slice of v_mfma_f32_32x32x16 from a 32x32 accumulator: the lane
// half hf holds accumulator rows 8g + 4hf + r (g = 0, 1; r = 0..3) of the
// slice, so storing the operand with bits 2 and 3 of k swapped makes those
// 8 rows the lane's 8 contiguous k values (slots 8hf .. 8hf + 7).
__device__ __forceinline__ int mfma_slot16(int k) {
  return (k & ~15) | (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// ---- LDS DMA and explicit waits (gfx950)

// s_waitcnt immediate: vmcnt <= n, expcnt and lgkmcnt unconstrained (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until this wavefront's LDS reads have returned (lgkmcnt = 0; vmcnt and
// expcnt unconstrained).  Needed before the barrier that releases a stage for
// overwriting: the compiler may otherwise consume the last fragment reads
// (and so wait for them) only after the barrier.
__device__ __forceinline__ void wait_lds_reads() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier without a memory fence or waits.  The compiler does not
// treat s_barrier as a memory operation, so empty asm statements with a
// memory clobber on both sides stop it from moving LDS accesses across; the
// waits the barrier needs are issued explicitly before it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS byte offset of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// One 16-byte global -> LDS copy per lane: lane i writes LDS [lds + 16 i].
// Issued as inline assembly so the compiler does not treat every later LDS
// read as dependent on it (it cannot tell the two pipeline stages apart and
// would wait for all outstanding copies); completion is awaited explicitly
// with wait_vmcnt before the workgroup barrier that publishes a stage.  The
// instruction has no register result; the address VGPRs are read at issue.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}

}  // namespace vt
