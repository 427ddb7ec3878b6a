// Pieces shared by the two chunk-forward kernels (the per-chunk transform and
// the sequential state pass): operand access for the I/O dtype, wave-level
// ordering, and the inverse of a unit lower triangular 16x16 block.
#pragma once

#include "device_common.h"
#include "launchers.h"

namespace gdr {

constexpr int CH = 64;   // chunk length

template <int IO> struct Op;
template <> struct Op<IO_BF16> {
  typedef __bf16 T;
  typedef bf16x4 frag;
  static constexpr int PAD = 8;      // row stride 4 (mod 32) dwords: fewest LDS bank conflicts (measured)
  static __device__ __forceinline__ frag ld(const T* p) { return *reinterpret_cast<const frag*>(p); }
  // Fragment holding M[r0 + 4*lg + s][c0 + lr], s = 0..3, of a row-major tile M:
  // the gfx950 LDS transpose load gathers it from 16 lanes' 8-byte reads.
  static __device__ __forceinline__ frag ld_tr(const T* m, int ld, int r0, int c0, int lr, int lg) {
    const T* a = m + (r0 + 4 * lg + (lr >> 2)) * ld + c0 + 4 * (lr & 3);
    typedef __attribute__((ext_vector_type(4))) short v4s;
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(const_cast<T*>(a)));
    return __builtin_bit_cast(frag, x);
  }
  static __device__ __forceinline__ frag cvt(f32x4 x) { return to_bf16x4(x); }
  static __device__ __forceinline__ f32x4 f32(frag x) {
    f32x4 r;
    r[0] = static_cast<float>(x[0]); r[1] = static_cast<float>(x[1]);
    r[2] = static_cast<float>(x[2]); r[3] = static_cast<float>(x[3]);
    return r;
  }
  static __device__ __forceinline__ T from(float x) { return static_cast<__bf16>(x); }
  static __device__ __forceinline__ f32x4 mma2(f32x4 acc, frag a0, frag a1, frag b0, frag b1) {
    return mma_k32_bf16(acc, a0, a1, b0, b1);
  }
  static __device__ __forceinline__ f32x4 mma1(f32x4 acc, frag a, frag b) { return mma_k16_bf16(acc, a, b); }
};
template <> struct Op<IO_F32> {
  typedef float T;
  typedef f32x4 frag;
  static constexpr int PAD = 4;
  static __device__ __forceinline__ frag ld(const T* p) { return *reinterpret_cast<const frag*>(p); }
  static __device__ __forceinline__ frag ld_tr(const T* m, int ld, int r0, int c0, int lr, int lg) {
    frag f;
#pragma unroll
    for (int s = 0; s < 4; ++s) f[s] = m[(r0 + 4 * lg + s) * ld + c0 + lr];
    return f;
  }
  static __device__ __forceinline__ frag cvt(f32x4 x) { return x; }
  static __device__ __forceinline__ f32x4 f32(frag x) { return x; }
  static __device__ __forceinline__ T from(float x) { return x; }
  static __device__ __forceinline__ f32x4 mma2(f32x4 acc, frag a0, frag a1, frag b0, frag b1) {
    return mma_k16_f32(mma_k16_f32(acc, a0, b0), a1, b1);
  }
  static __device__ __forceinline__ f32x4 mma1(f32x4 acc, frag a, frag b) { return mma_k16_f32(acc, a, b); }
};

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// Workspace record of one (sequence, head, chunk), written by the per-chunk
// transform and read by the state pass.  Two 64x64 matrices are kept as their
// ten 16x16 blocks on one side of the diagonal, block u = R(R+1)/2 + J for
// J <= R, each block row-major, in the I/O dtype:
//   T region: block u holds (T_RJ)^T, the transpose of block (R, J) of
//             T = (I + A)^{-1} (lower triangular);
//   P region: block u holds P_RJ of the masked score matrix (lower triangular;
//             written only where the state pass reads it: per-channel gate and
//             fp32 I/O);
// then six fp32 rows of 64 factors: with no gate or a scalar gate the per-row
// beta, e^{g_read}, e^{g}, e^{g_63 - g}, e^{g_63}, g; with a per-channel gate
// beta (row 0) and the per-channel decay e^{g_63} of the chunk (from row 1 on,
// d_k values).  With bf16 I/O and a per-channel gate the record goes on with the
// three decayed operands of the state pass, each row-major [64][d_k] in bf16:
// k e^{g_read}, q e^{g}, k e^{g_63 - g} (every factor is at most 1).
template <int ESZ>
struct WsRec {
  static constexpr int BLK = 256;                        // elements per 16x16 block
  static constexpr uint32_t T_OFF = 0;
  static constexpr uint32_t P_OFF = 10 * BLK * ESZ;
  static constexpr uint32_t F_OFF = 20 * BLK * ESZ;
  static constexpr int NF = 6;
  static constexpr uint32_t BYTES = F_OFF + NF * CH * 4;
  static constexpr uint32_t X_OFF = BYTES;               // decayed operands (bf16, per-channel gate)
  // byte offset of element (a, b) of block (R, J)
  static __device__ __forceinline__ uint32_t at(int R, int J, int a, int b) {
    return static_cast<uint32_t>(((R * (R + 1) / 2 + J) * BLK + a * 16 + b) * ESZ);
  }
};

// Per-channel gate: the transform splits each decay e^{g_r - g_j} at the first row
// of a 16-row block into a factor <= 1 on one operand and a factor >= 1 on the
// other, and the literal form's first row reads e^{g_{r-1} - g_16R} >= 1.  fp32
// (and bf16) hold e^x up to x ~ 88.7, and a factor below e^-SPLIT_MAX meeting one
// above e^+SPLIT_MAX loses at most e^-87.3 * e^SPLIT_MAX of a product to
// denormals.  A chunk in which some channel decays by more than e^-SPLIT_MAX
// inside one block (or within the row before a block) is marked in its record and
// its T and P blocks are formed again by chunk_prep_generic_kernel, which takes
// every decay as one exponential of a non-positive exponent.
constexpr float SPLIT_MAX = 64.f;
// Byte offset in a record of that mark (fp32; 1 = formed by the generic kernel).
// Row 5 of the factor rows is unused with a per-channel gate (d_k <= 128).
template <int ESZ>
__host__ __device__ constexpr uint32_t rec_flag_off() { return WsRec<ESZ>::F_OFF + 5 * CH * 4; }

// Bytes of one record for the I/O type, gate and d_k.
__host__ __device__ constexpr uint32_t rec_bytes(int io, int gate, int dk) {
  return io == IO_BF16 ? WsRec<2>::BYTES + (gate == GATE_CHANNEL ? 3u * CH * dk * 2u : 0u) : WsRec<4>::BYTES;
}

// Where one (sequence b, head h) lies.  Fixed-length batches ([B, T, H, .]
// tensors): tokens b T .. b T + T - 1, records (b H + h) ceil(T / 64) onwards.
// Packed sequences (p.cu set; [1, T, H, .] tensors, p.B sequences): tokens
// cu[b] .. cu[b+1] - 1, clamped to [0, T] with a length of at least 0 so that a
// malformed offset table still stays inside the tensors, and records
// h p.nslots + floor(cu[b] / 64) + b onwards.  For non-decreasing offsets those
// record ranges are disjoint (sequence b's last chunk lies below b + 1's first
// slot) and end below h p.nslots + ceil(T / 64) + B - 1.
struct SeqSpan {
  int64_t t0, len, rec0;
};
// A wave-uniform 64-bit value, kept in scalar registers (buffer descriptors built
// from values the compiler cannot prove uniform go through waterfall loops).
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ int64_t seq_start(const ChunkParams& p, int64_t b) {
  const int64_t a = p.cu[b];
  return a < 0 ? 0 : (a > p.T ? p.T : a);
}
__device__ __forceinline__ SeqSpan seq_span(const ChunkParams& p, int64_t b, int64_t h) {
  if (!p.cu) return SeqSpan{b * p.T, p.T, (b * p.H + h) * ((p.T + CH - 1) / CH)};
  const int64_t a = seq_start(p, b);
  int64_t e = p.cu[b + 1];
  e = e < a ? a : (e > p.T ? p.T : e);
  return SeqSpan{uni64(a), uni64(e - a), uni64(h * p.nslots + a / CH + b)};
}
// Tasks of the per-chunk transform, head fastest: fixed-length batches
// (b, chunk, h) for B H ceil(T / 64) tasks; packed sequences (slot, h) for
// H nslots tasks, the sequence of a slot found by bisection over the slot bases.
// Returns false for a task with no chunk (a slot past the end of its sequence).
__device__ __forceinline__ int64_t prep_tasks_fixed(const ChunkParams& p) { return p.B * p.H * ((p.T + CH - 1) / CH); }
__device__ __forceinline__ bool prep_task(const ChunkParams& p, int64_t task, int64_t& b, int64_t& n, int64_t& h) {
  h = task % p.H;
  if (!p.cu) {
    const int64_t nch = (p.T + CH - 1) / CH;
    n = (task / p.H) % nch;
    b = task / (p.H * nch);
    return true;
  }
  const int64_t slot = task / p.H;
  int64_t lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (seq_start(p, mid) / CH + mid <= slot) lo = mid; else hi = mid - 1;
  }
  b = uni64(lo);
  const SeqSpan s = seq_span(p, b, h);
  n = uni64(slot - (s.t0 / CH + b));
  return n >= 0 && n * CH < s.len;
}

// The record index of transform task `task` when every lane has a task of its own
// (prep_task keeps its results wave-uniform).  Same mapping: fixed-length
// (b H + h) ceil(T / 64) + n; packed sequences h nslots + slot.  False for a task
// with no chunk.
__device__ __forceinline__ bool task_record(const ChunkParams& p, int64_t task, int64_t& rec) {
  const int64_t h = task % p.H;
  if (!p.cu) {
    const int64_t nch = (p.T + CH - 1) / CH;
    const int64_t n = (task / p.H) % nch, b = task / (p.H * nch);
    rec = (b * p.H + h) * nch + n;
    return true;
  }
  const int64_t slot = task / p.H;
  int64_t lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (seq_start(p, mid) / CH + mid <= slot) lo = mid; else hi = mid - 1;
  }
  const int64_t a = seq_start(p, lo);
  int64_t e = p.cu[lo + 1];
  e = e < a ? a : (e > p.T ? p.T : e);
  const int64_t n = slot - (a / CH + lo);
  rec = h * p.nslots + slot;
  return n >= 0 && n * CH < e - a;
}

// Block (R, J), J <= R, of the ten-block order above.
__device__ __forceinline__ void tri_block(int u, int& R, int& J) {
  R = (u >= 1) + (u >= 3) + (u >= 6);
  J = u - R * (R + 1) / 2;
}

__device__ __forceinline__ int strict_pair(int R, int J) { return R * (R - 1) / 2 + J; }

// Ordering point for LDS traffic between the lanes of one wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// (I + N)^{-1} of a strictly lower 16x16 block N held as an accumulator tile, by
// the finite Neumann product (I - N)(I + N^2)(I + N^4)(I + N^8) (N^16 = 0), on
// fp32 MFMA.  `scr` is this wave's 16x16 fp32 scratch, used to turn an
// accumulator tile into a row-major A operand.
__device__ __forceinline__ f32x4 unit_lower_inverse(f32x4 N, float* scr, int lr, int lg) {
  constexpr int LSC = 20;
  auto put = [&](f32x4 M) {
#pragma unroll
    for (int s = 0; s < 4; ++s) scr[(4 * lg + s) * LSC + lr] = M[s];
  };
  auto rows = [&]() -> f32x4 { return *reinterpret_cast<const f32x4*>(scr + lr * LSC + 4 * lg); };
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 Y;
#pragma unroll
  for (int s = 0; s < 4; ++s) Y[s] = (4 * lg + s == lr ? 1.f : 0.f) - N[s];
  put(N);
  wave_sync();
  f32x4 a = rows();
  wave_sync();
  f32x4 P = mma_k16_f32(zero, a, N);          // N^2
  put(P);
  wave_sync();
  a = rows();
  wave_sync();
  Y = mma_k16_f32(Y, a, Y);                   // (I + N^2)(I - N)
  P = mma_k16_f32(zero, a, P);                // N^4
  put(P);
  wave_sync();
  a = rows();
  wave_sync();
  Y = mma_k16_f32(Y, a, Y);
  P = mma_k16_f32(zero, a, P);                // N^8
  put(P);
  wave_sync();
  a = rows();
  wave_sync();
  return mma_k16_f32(Y, a, Y);
}

// (I + N)^{-1} of a strictly lower 16x16 block N, in registers, for one wave.
// N and Nt are the accumulator tiles of N and of N^T.  An accumulator tile of X
// fed back as the B operand of a product stands for X, and as the A operand for
// X^T, so both orientations of every power are formed side by side:
//     D = (I - N)(I + N^2)(I + N^4)(I + N^8)   (N^16 = 0; the factors commute)
// Returns D in D and D^T in Dt (both accumulator tiles); 12 products on the
// MFMA of the I/O dtype with fp32 accumulation.
template <class O>
__device__ __forceinline__ void unit_lower_inverse_pair(f32x4 N, f32x4 Nt, f32x4& D, f32x4& Dt, int lr, int lg) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 Y, Yt;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const float id = 4 * lg + s == lr ? 1.f : 0.f;
    Y[s] = id - N[s];
    Yt[s] = id - Nt[s];
  }
  const f32x4 N2 = O::mma1(z, O::cvt(Nt), O::cvt(N));      // N N
  const f32x4 N2t = O::mma1(z, O::cvt(N), O::cvt(Nt));     // N^T N^T
  Y = O::mma1(Y, O::cvt(N2t), O::cvt(Y));                  // (I + N^2) Y
  Yt = O::mma1(Yt, O::cvt(N2), O::cvt(Yt));                // (Y (I + N^2))^T
  const f32x4 N4 = O::mma1(z, O::cvt(N2t), O::cvt(N2));
  const f32x4 N4t = O::mma1(z, O::cvt(N2), O::cvt(N2t));
  Y = O::mma1(Y, O::cvt(N4t), O::cvt(Y));
  Yt = O::mma1(Yt, O::cvt(N4), O::cvt(Yt));
  const f32x4 N8 = O::mma1(z, O::cvt(N4t), O::cvt(N4));
  const f32x4 N8t = O::mma1(z, O::cvt(N4), O::cvt(N4t));
  D = O::mma1(Y, O::cvt(N8t), O::cvt(Y));
  Dt = O::mma1(Yt, O::cvt(N8), O::cvt(Yt));
}

}  // namespace gdr
