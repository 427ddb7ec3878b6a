// Shared pieces of the backward kernels (chunk_bwd.hip, chunk_bwd_chan.hip): operand
// fragments of 16x16 MFMA tiles read from LDS, LDS row strides, the (sequence, head)
// slices of the token tensors, and fixed-order lane sums.
//
// Operand fragments (lane l: lr = l % 16, lg = l / 16):
//   rowf(M, ld, x0, k0) = M[x0 + lr][k0 + 4 lg + s]   (8-byte LDS read)
//   colf(M, ld, k0, x0) = M[k0 + 4 lg + s][x0 + lr]   (LDS transpose read)
// For C = A B an A fragment is A[m0 + lr][k0 + 4 lg + s] and a B fragment
// B[k0 + 4 lg + s][n0 + lr].  mma(a, b) leaves C[m0 + 4 lg + s][n0 + lr] in the lane
// (the "column" form, whose tiles feed the next product as B fragments); mma(b, a)
// leaves C[m0 + lr][n0 + 4 lg + s] (the "row" form: one row per lane, four adjacent
// columns, written with one 8-byte store).
#pragma once

#include "chunk_common.h"

namespace gdr {
namespace {


typedef Op<IO_BF16> O;
typedef __bf16 T;
typedef bf16x4 frag;
typedef WsRec<2> W;

__device__ __forceinline__ frag rowf(const T* m, int ld, int x0, int k0, int lr, int lg) {
  return O::ld(m + (x0 + lr) * ld + k0 + 4 * lg);
}
__device__ __forceinline__ frag colf(const T* m, int ld, int k0, int x0, int lr, int lg) {
  return O::ld_tr(m, ld, k0, x0, lr, lg);
}
__device__ __forceinline__ void st_row(T* m, int ld, int r, int c, f32x4 x) {
  *reinterpret_cast<frag*>(m + r * ld + c) = to_bf16x4(x);
}
__device__ __forceinline__ void buf_store2(uint16_t x, rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b16(x, r, voff, soff, 0);
}
__device__ __forceinline__ u32x2 bits8(f32x4 x) { return __builtin_bit_cast(u32x2, to_bf16x4(x)); }
// A 16-byte piece into a tile whose rows are 8-byte aligned: two 8-byte stores.
__device__ __forceinline__ void put16(T* dst, u32x4 x) {
  u32x2* d = reinterpret_cast<u32x2*>(dst);
  d[0] = u32x2{x[0], x[1]};
  d[1] = u32x2{x[2], x[3]};
}

// LDS row strides (bf16 elements) by how a tile is read, after the rates measured
// for the forward on gfx950: 8-byte row fragments run fastest when a row is 2 or 6
// (mod 8) dwords long, transpose reads when it is 8 (mod 32) dwords; a tile read both
// ways takes 6 (mod 8).
constexpr int ld_row(int w) { return w + 4; }     // rows only
constexpr int ld_tr(int w) { return w + 16; }     // transposed only (w = 64, 128)
constexpr int ld_both(int w) { return w + 12; }   // both

// Buffers over one (sequence, head) slice of a [B, T, H, width] tensor; the range
// ends after the last token, so rows past it read as zero and their stores drop.
struct Slice {
  int64_t row0;
  uint32_t span;
  __device__ __forceinline__ rsrc_t rs(const void* base, int width) const {
    return make_rsrc(static_cast<const uint16_t*>(base) + row0 * width, span * width * 2);
  }
};
// One (sequence, head): its token rows, chunks, and first record slot (the per-chunk
// records and both sets of chunk states are addressed by the same slots).
// Fixed-length batches: [B, T, H, .] tensors; packed sequences (f.cu set): tokens
// cu[b] .. cu[b+1] - 1 of [1, T, H, .] tensors (see seq_span).
struct BwdSeq {
  Slice sl;
  int64_t nch, rec0;
};
__device__ __forceinline__ BwdSeq bwd_seq_of(const ChunkParams& f, int64_t bb, int64_t hh) {
  const SeqSpan sp = seq_span(f, bb, hh);
  return BwdSeq{Slice{sp.t0 * f.H + hh, static_cast<uint32_t>(sp.len > 0 ? (sp.len - 1) * f.H + 1 : 0)},
                (sp.len + CH - 1) / CH, sp.rec0};
}

// Sum over the 16 lanes of a row (lanes with one lg), returned to all of them;
// the pairing is fixed, so the result is the same on every run.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0x128>(v);   // row_ror:8
  v += dpp<0x124>(v);   // row_ror:4
  v += dpp<0x122>(v);   // row_ror:2
  v += dpp<0x121>(v);   // row_ror:1
  return v;
}
// Sum over the four lanes with one lr (lanes lr, lr + 16, lr + 32, lr + 48).
__device__ __forceinline__ float lg_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace
}  // namespace gdr
