// Device helpers shared by the gfx950 kernels: I/O dtype traits and MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

enum IoType { IO_F32 = 0, IO_BF16 = 1 };
enum GateKind { GATE_NONE = 0, GATE_SCALAR = 1, GATE_CHANNEL = 2 };
// Kernel variants (never values of the C ABI's gate): a separate write key k~ for
// the state write (the right-preconditioned delta rule), without a gate or with a
// scalar gate.  (The per-channel gate takes the write key through its transform's
// operands and keeps GATE_CHANNEL.)
constexpr int GATE_WKEY = 3;
constexpr int GATE_WKEY_SCALAR = 4;
__host__ __device__ constexpr bool gate_scalar(int g) { return g == GATE_SCALAR || g == GATE_WKEY_SCALAR; }
__host__ __device__ constexpr bool gate_wkey(int g) { return g == GATE_WKEY || g == GATE_WKEY_SCALAR; }

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (the conversion gfx950 performs in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

// Element access for the I/O dtype.
template <int IO> struct Io;
template <> struct Io<IO_F32> {
  typedef float elem;
  static __device__ __forceinline__ float load(const elem* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(elem* p, int64_t i, float x) { p[i] = x; }
};
template <> struct Io<IO_BF16> {
  typedef uint16_t elem;
  static __device__ __forceinline__ float load(const elem* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
  static __device__ __forceinline__ void store(elem* p, int64_t i, float x) { p[i] = f32_to_bf16_bits(x); }
};

// ---------------------------------------------------------------------------
// MFMA building block.  All products are 16x16 output tiles, accumulated in
// fp32, in the gfx950 accumulator layout: lane l holds column n = l % 16 and
// rows 4*(l/16) + s, s = 0..3.
//
// A k-extent of 16 is one "sub-block"; within a sub-block, lane group g = l/16
// supplies k = 4g .. 4g+3 (for A: row m = l % 16; for B: column n = l % 16).
// This is exactly what an accumulator tile holds, so an fp32 accumulator tile
// can be fed back as the B operand of the next product after conversion.
//
// bf16: two sub-blocks form one v_mfma_f32_16x16x32_bf16 (the instruction's
//       k-order is permuted consistently on A and B, which leaves the sum
//       unchanged).  A lone sub-block is the same instruction with a zero upper
//       half: every bf16 accumulation chain uses one opcode.  (Feeding the result
//       of a 16x16x32 product into a 16x16x16 product's accumulator input gave
//       wrong values on gfx950 with this compiler; the legacy 16x16x16 opcode
//       also runs at half rate, so the padded form costs nothing.)
// f32:  one sub-block is four v_mfma_f32_16x16x4_f32, one per k = 4g + s.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
  bf16x4 r;
  r[0] = static_cast<__bf16>(x[0]);
  r[1] = static_cast<__bf16>(x[1]);
  r[2] = static_cast<__bf16>(x[2]);
  r[3] = static_cast<__bf16>(x[3]);
  return r;
}

__device__ __forceinline__ f32x4 mma_k32_bf16(f32x4 acc, bf16x4 a_lo, bf16x4 a_hi, bf16x4 b_lo,
                                               bf16x4 b_hi) {
  bf16x8 a = __builtin_shufflevector(a_lo, a_hi, 0, 1, 2, 3, 4, 5, 6, 7);
  bf16x8 b = __builtin_shufflevector(b_lo, b_hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma_k16_bf16(f32x4 acc, bf16x4 a, bf16x4 b) {
  const bf16x4 z = {};
  return mma_k32_bf16(acc, a, z, b, z);
}

__device__ __forceinline__ f32x4 mma_k16_f32(f32x4 acc, f32x4 a, f32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
  return acc;
}

// ---------------------------------------------------------------------------
// Buffer resources: a base address plus a byte range.  Loads past the range
// return zero and stores past it are dropped, which is how the kernels handle
// the ragged end of a sequence without per-lane guards.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // third descriptor word: 32-bit data format, as for untyped gfx9 buffer access
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint16_t buf_load2(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store8(u32x2 x, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(x, r, voff, soff, 0);
}
// A streaming store (non-temporal): data read back only by a later kernel.
__device__ __forceinline__ void buf_store8_nt(u32x2 x, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(x, r, voff, soff, 2);
}
__device__ __forceinline__ void buf_store16(u32x4 x, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, soff, 0);
}

}  // namespace gdr
