// Chunkwise-parallel forward of the gated delta rule on gfx950 (one fused kernel).
//
// Method: "Moonshot AI's New Attention Architecture: Key Innovations Explained",
// §3 Hardware-Friendly Algorithm -- the sequence is cut into chunks of C = 64
// tokens; inside a chunk the work is dense (lower-triangular) matrix products,
// between chunks only the d_k x d_v state is passed on; §5 Practical
// Considerations -- the cumulative gate is kept in the log domain.  The update
// being computed is the per-channel gated delta rule of §2 of the same page
// (key-major state S, d_k rows, d_v columns):
//     S_t = (I - beta_t k_t k_t^T) diag(a_t) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t.
//
// Per chunk (rows r = 0..63, g_r = inclusive running sum of log a inside the chunk,
// S the state entering the chunk):
//   A     = strict_lower( diag(beta) (K*e^{g_read}) (K*e^{-g})^T )     g_read = g (decay
//           before the erase) or g_{r-1} (erase reads the undecayed state)
//   W     = (I + A)^{-1} diag(beta) (K*e^{g_read}),   U = (I + A)^{-1} diag(beta) V
//   Delta = U - W S
//   O     = (Q*e^{g}) S + lower_incl( (Q*e^{g}) (K*e^{-g})^T ) Delta
//   S'    = diag(e^{g_63}) S + (K*e^{g_63 - g})^T Delta
// (the correction terms W, U and the two state/output equations of §3; the
// query/key decay factors as derived from the §2 update).
//
// Work decomposition.  One workgroup of NW waves owns one (batch, head, d_v tile
// of 16*NW columns) and walks the chunks in order.  Wave w owns 16 state
// columns: its slice of S (d_k x 16, fp32) lives in MFMA accumulators for the
// whole sequence.  An accumulator tile (lane l: column l%16, rows 4(l/16)+s) is
// the operand layout of the next product, so W*S, the output and the state
// update chain through registers.  The d_v-independent per-chunk work (log-gate
// scan, the 16x16 blocks of A and of the masked score matrix P, the four
// diagonal 16x16 inverses) is shared by the waves through LDS.  (I + A)^{-1} is
// never formed: each wave solves for its own columns of W and U by forward
// substitution over the four 16-row blocks.  The next chunk's q, k, v, beta and
// log-gate are loaded into registers (16-byte loads) while the current chunk
// computes.
//
// Gates.  With no gate or a scalar gate the decay factors are per row and per
// column of the 64x64 intra-chunk matrices, so the products run on the raw
// q, k, v tiles and the factors are applied to the results (A and P element by
// element, the output and Delta row by row).  A per-channel gate sits inside
// the d_k contraction, so decayed operands are built first; for the score
// matrices the factor e^{g_r - g_j} is split at the first row of each 16-row
// block (e^{g_r - g_16R} on rows, e^{g_16J - g_j} on columns, e^{g_16R - g_16J} on
// the column operand of blocks below the diagonal), so no operand exceeds the
// decay accumulated over 15 tokens.
//
// Products run on bf16 MFMA with fp32 accumulation for bf16 I/O and on fp32
// MFMA for fp32 I/O; the state stays fp32.
#include <type_traits>

#include "device_common.h"
#include "launchers.h"

namespace gdr {

constexpr int CH = 64;   // chunk length

template <int IO> struct Op;
template <> struct Op<IO_BF16> {
  typedef __bf16 T;
  typedef bf16x4 frag;
  static constexpr int PAD = 8;
  static __device__ __forceinline__ frag ld(const T* p) { return *reinterpret_cast<const frag*>(p); }
  static __device__ __forceinline__ frag cvt(f32x4 x) { return to_bf16x4(x); }
  static __device__ __forceinline__ f32x4 f32(frag x) {
    f32x4 r;
    r[0] = static_cast<float>(x[0]); r[1] = static_cast<float>(x[1]);
    r[2] = static_cast<float>(x[2]); r[3] = static_cast<float>(x[3]);
    return r;
  }
  static __device__ __forceinline__ T from(float x) { return static_cast<__bf16>(x); }
  static __device__ __forceinline__ float to(T x) { return static_cast<float>(x); }
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
  static __device__ __forceinline__ frag cvt(f32x4 x) { return x; }
  static __device__ __forceinline__ f32x4 f32(frag x) { return x; }
  static __device__ __forceinline__ T from(float x) { return x; }
  static __device__ __forceinline__ float to(T x) { return x; }
  static __device__ __forceinline__ f32x4 mma2(f32x4 acc, frag a0, frag a1, frag b0, frag b1) {
    return mma_k16_f32(mma_k16_f32(acc, a0, b0), a1, b1);
  }
  static __device__ __forceinline__ f32x4 mma1(f32x4 acc, frag a, frag b) { return mma_k16_f32(acc, a, b); }
};

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// LDS layout (bytes).  Row-major [64][DK] tiles use stride LDK, transposed
// [*][64] tiles stride LCH; both carry padding against bank conflicts.
template <int IO, int GATE, int DK, int NW>
struct Layout {
  typedef typename Op<IO>::T T;
  static constexpr bool RAW = GATE != GATE_CHANNEL;   // products on raw q, k, v
  static constexpr int PAD = Op<IO>::PAD;
  static constexpr int LDK = DK + PAD;
  static constexpr int LCH = CH + PAD;
  static constexpr int LA = CH + 4;
  static constexpr int LXI = 16 + PAD;
  static constexpr int LSC = 20;                       // per-wave 16x16 fp32 scratch stride
  static constexpr int DVT = 16 * NW;
  static constexpr int NSEG = (64 * NW) / DK > 0 ? (64 * NW) / DK : 1;
  static constexpr size_t RM = size_t(CH) * LDK * sizeof(T);      // [64][DK]
  static constexpr size_t TR = size_t(DK) * LCH * sizeof(T);      // [DK][64]
  static constexpr size_t A_B = size_t(CH) * LA * 4;
  static constexpr size_t P_B = size_t(CH) * LCH * sizeof(T);
  static constexpr size_t XI_B = size_t(CH) * LXI * sizeof(T);
  static constexpr size_t VT_B = size_t(DVT) * LCH * sizeof(T);
  static constexpr size_t SC_B = size_t(NW) * 16 * LSC * 4;
  // common regions
  static constexpr size_t OFF_K = 0;                     // raw k (channel: X_K in place), then W
  static constexpr size_t OFF_Q = OFF_K + RM;            // raw q (channel: X_Q in place)
  static constexpr size_t OFF_VT = OFF_Q + RM;           // raw v tile, transposed
  static constexpr size_t OFF_XI = OFF_VT + VT_B;        // inverses of the diagonal blocks
  static constexpr size_t OFF_SC = OFF_XI + XI_B;        // per-wave scratch of the inversion
  static constexpr size_t OFF_X = OFF_SC + SC_B;         // gate-dependent regions start here
  // raw gates
  static constexpr size_t R_KT = OFF_X;                  // k transposed
  static constexpr size_t R_A = R_KT + TR;
  static constexpr size_t R_P = R_A + A_B;
  static constexpr size_t R_SMALL = R_P + P_B;           // beta, g, g_read, e_w, e_o, e_d, gamma
  static constexpr size_t R_TOTAL = R_SMALL + 7 * CH * 4;
  // per-channel gate
  static constexpr size_t C_Y = OFF_X;                   // column operand of the score blocks
  static constexpr size_t C_QH = C_Y + RM;
  static constexpr size_t C_KRT = C_QH + RM;
  static constexpr size_t C_KDT = C_KRT + TR;
  static constexpr size_t C_G = C_KDT + TR;              // g [64][DK] fp32, then A and P
  static constexpr size_t C_G_B = cmax(size_t(CH) * DK * 4, A_B + P_B);
  static constexpr size_t C_BETA = C_G + C_G_B;
  static constexpr size_t C_GAM = C_BETA + CH * 4;
  static constexpr size_t C_M = C_GAM + DK * 4;
  static constexpr size_t C_TOT = C_M + 6 * DK * 4;
  static constexpr size_t C_TOTAL = C_TOT + NSEG * DK * 4;
  static constexpr size_t TOTAL = RAW ? R_TOTAL : C_TOTAL;
};

__device__ __forceinline__ int strict_pair(int R, int J) { return R * (R - 1) / 2 + J; }

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// x if keep else 0, component by component (a whole-vector select can be lowered
// through private memory)
__device__ __forceinline__ uint4 keep_or_zero(bool keep, uint4 x) {
  const uint32_t m = keep ? 0xffffffffu : 0u;
  return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
}

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

template <int IO, int GATE, int DK, int NW>
__global__ __launch_bounds__(NW * 64) void chunk_fwd_kernel(ChunkParams p, int n_tiles) {
  typedef Op<IO> O;
  typedef typename O::T T;
  typedef typename O::frag frag;
  typedef typename Io<IO>::elem elem;
  typedef Layout<IO, GATE, DK, NW> L;
  constexpr bool RAW = L::RAW;
  constexpr int NT = NW * 64;
  constexpr int DVT = 16 * NW;
  constexpr int DKT = DK / 16;
  constexpr int CBW = DKT / NW;          // 16-channel blocks of W solved per wave
  constexpr int LDK = L::LDK, LCH = L::LCH, LA = L::LA, LXI = L::LXI;
  constexpr int EPV = 16 / int(sizeof(elem));   // elements per 16-byte load
  constexpr int KROW = DK / EPV;
  constexpr int KV = CH * KROW / NT;            // row-major 16-byte pieces of a k (q) tile per thread
  constexpr int KTT = RAW ? DK * 8 / NT : 1;    // 8-row column runs of k^T per thread
  constexpr int VTT = DVT * 8 / NT;             // 8-row column runs of v^T per thread
  static_assert(CBW >= 1 && CBW * NW == DKT, "channel blocks must split over waves");
  static_assert(KV * NT == CH * KROW && VTT * NT == DVT * 8 && (!RAW || KTT * NT == DK * 8), "even split");
  static_assert(L::TOTAL <= 163840, "LDS budget");

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  T* sK = reinterpret_cast<T*>(smem + L::OFF_K);
  T* sQ = reinterpret_cast<T*>(smem + L::OFF_Q);
  T* sVT = reinterpret_cast<T*>(smem + L::OFF_VT);
  T* sXi = reinterpret_cast<T*>(smem + L::OFF_XI);
  float* sScr = reinterpret_cast<float*>(smem + L::OFF_SC);
  T* sW = sK;                       // k is dead once A and P are formed
  // raw-gate regions
  T* sKT = reinterpret_cast<T*>(smem + L::R_KT);
  float* sSmall = reinterpret_cast<float*>(smem + L::R_SMALL);
  float* sBr = sSmall;              // beta
  float* sGr = sSmall + CH;         // g
  float* sGrd = sSmall + 2 * CH;    // g_read
  float* sEw = sSmall + 3 * CH;     // beta e^{g_read}   (right-hand side of W)
  float* sEo = sSmall + 4 * CH;     // e^{g}             (output rows)
  float* sEd = sSmall + 5 * CH;     // e^{g_63 - g}      (Delta rows in the state update)
  float* sGamR = sSmall + 6 * CH;   // e^{g_63}
  // per-channel regions
  T* sY = reinterpret_cast<T*>(smem + L::C_Y);
  T* sQh = reinterpret_cast<T*>(smem + L::C_QH);
  T* sKrT = reinterpret_cast<T*>(smem + L::C_KRT);
  T* sKdT = reinterpret_cast<T*>(smem + L::C_KDT);
  float* sG = reinterpret_cast<float*>(smem + L::C_G);
  float* sBc = reinterpret_cast<float*>(smem + L::C_BETA);
  float* sGamC = reinterpret_cast<float*>(smem + L::C_GAM);
  float* sM = reinterpret_cast<float*>(smem + L::C_M);
  float* sTot = reinterpret_cast<float*>(smem + L::C_TOT);
  float* sA = RAW ? reinterpret_cast<float*>(smem + L::R_A) : sG;
  T* sP = RAW ? reinterpret_cast<T*>(smem + L::R_P) : reinterpret_cast<T*>(smem + L::C_G + L::A_B);
  float* sBeta = RAW ? sBr : sBc;

  const elem* gq = static_cast<const elem*>(p.q);
  const elem* gk = static_cast<const elem*>(p.k);
  const elem* gv = static_cast<const elem*>(p.v);
  const elem* gbeta = static_cast<const elem*>(p.beta);
  const elem* gla = static_cast<const elem*>(p.log_a);
  elem* go = static_cast<elem*>(p.o);

  // Block -> (head, d_v tile).  Consecutive logical blocks land on one XCD (the
  // hardware deals block ids round-robin over 8 XCDs), so the tiles of one head
  // share that XCD's L2 for their common q, k, log_a reads.
  const int nblk = gridDim.x;
  int lb = blockIdx.x;
  if ((nblk & 7) == 0) lb = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int64_t bh = lb / n_tiles;
  const int tile = lb % n_tiles;
  const int64_t bb = bh / p.H, hh = bh % p.H;
  const int dv = p.d_v;
  const int col0 = tile * DVT;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int scol = col0 + 16 * wave + lr;   // this lane's state column

  auto tok = [&](int64_t t) -> int64_t { return (bb * p.T + t) * p.H + hh; };

  // State slice: S[t][s] = S[16t + 4lg + s][scol].
  f32x4 S[DKT];
#pragma unroll
  for (int t = 0; t < DKT; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      S[t][s] = p.S0 ? p.S0[(bh * DK + 16 * t + 4 * lg + s) * dv + scol] : 0.f;

  // ---- register prefetch of one chunk's inputs ----------------------------------
  // Rows past the end of the sequence are read from the last valid row (so no
  // load needs a guard and none stalls the issuing wave) and zeroed when the
  // registers are written to LDS.
  constexpr int RW = 8 * int(sizeof(elem)) / 4;         // 32-bit words in an 8-element run
  uint4 pk[KV], pq[KV], pl[GATE == GATE_CHANNEL ? KV : 1];
  uint32_t pkt[KTT][RW], pvt[VTT][RW];
  // element e of a 16-byte piece / of an 8-element run, as float
  auto elem_of = [&](const uint32_t* w, int e) -> float {
    if constexpr (IO == IO_BF16) return bf16_bits_to_f32(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1))));
    else return __uint_as_float(w[e]);
  };
  auto load_run = [&](uint32_t* w, const elem* base, int64_t t0m, int row0, int last, int64_t stride)
      __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = row0 + e;
      const elem x = base[tok(t0m + (row < last ? row : last)) * stride];
      if constexpr (IO == IO_BF16) {
        if (e & 1) w[e >> 1] |= uint32_t(x) << 16; else w[e >> 1] = uint32_t(x);
      } else {
        w[e] = __float_as_uint(x);
      }
    }
  };
  float pb = 0.f, pls = 0.f;
  auto prefetch = [&](int64_t m) __attribute__((always_inline)) {
    const int64_t t0m = m * CH;
    const int last = static_cast<int>(p.T - t0m < CH ? p.T - t0m : CH) - 1;
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int seg = tid + v * NT, row = seg / KROW, c = (seg % KROW) * EPV;
      const int64_t off = tok(t0m + (row < last ? row : last)) * DK + c;
      pk[v] = ldg16(gk + off);
      pq[v] = ldg16(gq + off);
      if constexpr (GATE == GATE_CHANNEL) pl[v] = ldg16(gla + off);
    }
    if constexpr (RAW) {
#pragma unroll
      for (int j = 0; j < KTT; ++j) {
        const int task = tid + j * NT, i = task % DK, rg = task / DK;
        load_run(pkt[j], gk + i, t0m, 8 * rg, last, DK);
      }
    }
#pragma unroll
    for (int j = 0; j < VTT; ++j) {
      const int task = tid + j * NT, c = task % DVT, rg = task / DVT;
      load_run(pvt[j], gv + col0 + c, t0m, 8 * rg, last, dv);
    }
    if (tid < CH) {
      const int row = tid < last ? tid : last;
      pb = Io<IO>::load(gbeta, tok(t0m + row));
      if constexpr (GATE == GATE_SCALAR) pls = Io<IO>::load(gla, tok(t0m + row));
    }
  };
  auto put_run = [&](T* dst, const uint32_t* w, int row0, int nrows) __attribute__((always_inline)) {   // 8 rows of one column
    frag f0, f1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f0[e] = O::from(row0 + e < nrows ? elem_of(w, e) : 0.f);
      f1[e] = O::from(row0 + 4 + e < nrows ? elem_of(w, e + 4) : 0.f);
    }
    *reinterpret_cast<frag*>(dst) = f0;
    *reinterpret_cast<frag*>(dst + 4) = f1;
  };

  const int64_t nchunks = (p.T + CH - 1) / CH;
  if (nchunks > 0) prefetch(0);

  for (int64_t n = 0; n < nchunks; ++n) {
    const int64_t t0 = n * CH;
    const int nrows = static_cast<int>(p.T - t0 < CH ? p.T - t0 : CH);

    // ---- (0) chunk from registers into LDS, per-chunk log-gate; next chunk's loads
    {
#pragma unroll
      for (int v = 0; v < KV; ++v) {
        const int seg = tid + v * NT, row = seg / KROW, c = (seg % KROW) * EPV;
        const bool live = row < nrows;
        *reinterpret_cast<uint4*>(sK + row * LDK + c) = keep_or_zero(live, pk[v]);
        *reinterpret_cast<uint4*>(sQ + row * LDK + c) = keep_or_zero(live, pq[v]);
        if constexpr (GATE == GATE_CHANNEL) {
          const uint32_t w[4] = {pl[v].x, pl[v].y, pl[v].z, pl[v].w};
#pragma unroll
          for (int j = 0; j < EPV; ++j) sG[row * DK + c + j] = live ? elem_of(w, j) : 0.f;
        }
      }
      if constexpr (RAW) {
#pragma unroll
        for (int j = 0; j < KTT; ++j) {
          const int task = tid + j * NT, i = task % DK, rg = task / DK;
          put_run(sKT + i * LCH + 8 * rg, pkt[j], 8 * rg, nrows);
        }
      }
#pragma unroll
      for (int j = 0; j < VTT; ++j) {
        const int task = tid + j * NT, c = task % DVT, rg = task / DVT;
        put_run(sVT + c * LCH + 8 * rg, pvt[j], 8 * rg, nrows);
      }
      if constexpr (RAW) {
        if (wave == 0) {            // inclusive scan of the log-gate over the chunk rows
          const bool live = lane < nrows;
          const float be = live ? pb : 0.f;
          float g = 0.f, gread = 0.f;
          if constexpr (GATE == GATE_SCALAR) {
            g = live ? pls : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
              const float y = __shfl_up(g, off);
              if (lane >= off) g += y;
            }
            const float gprev = __shfl_up(g, 1);
            gread = p.literal ? (lane == 0 ? 0.f : gprev) : g;
          }
          const float gC = __shfl(g, 63);
          sBr[lane] = be;
          sGr[lane] = g;
          sGrd[lane] = gread;
          sEw[lane] = be * __expf(gread);
          sEo[lane] = __expf(g);
          sEd[lane] = __expf(gC - g);
          if (lane == 0) sGamR[0] = __expf(gC);
        }
      } else {
        if (tid < CH) sBc[tid] = tid < nrows ? pb : 0.f;
      }
    }
    if (n + 1 < nchunks) prefetch(n + 1);
    __syncthreads();

    if constexpr (!RAW) {
      // per-channel scan over the rows of each channel
      constexpr int NSEG = L::NSEG, SEGL = CH / NSEG;
      if (tid < NSEG * DK) {
        const int i = tid % DK, seg = tid / DK;
        float acc = 0.f;
#pragma unroll 8
        for (int r = seg * SEGL; r < (seg + 1) * SEGL; ++r) {
          acc += sG[r * DK + i];
          sG[r * DK + i] = acc;
        }
        sTot[seg * DK + i] = acc;
      }
      if constexpr (NSEG > 1) {
        __syncthreads();
        if (tid < NSEG * DK) {
          const int i = tid % DK, seg = tid / DK;
          float pre = 0.f;
          for (int s2 = 0; s2 < seg; ++s2) pre += sTot[s2 * DK + i];
          if (seg > 0)
            for (int r = seg * SEGL; r < (seg + 1) * SEGL; ++r) sG[r * DK + i] += pre;
        }
      }
      __syncthreads();
      // decayed operands; X_K and X_Q overwrite the raw tiles in place
      for (int i = tid; i < DK; i += NT) {
        sGamC[i] = __expf(sG[(CH - 1) * DK + i]);
#pragma unroll
        for (int R = 1; R < 4; ++R)
#pragma unroll
          for (int J = 0; J < R; ++J)
            sM[strict_pair(R, J) * DK + i] = __expf(sG[16 * R * DK + i] - sG[16 * J * DK + i]);
      }
      for (int task = tid; task < CH * (DK / 4); task += NT) {
        const int r = task / (DK / 4), i0 = (task % (DK / 4)) * 4, R = r >> 4;
        const f32x4 kk = O::f32(O::ld(sK + r * LDK + i0));
        const f32x4 qq = O::f32(O::ld(sQ + r * LDK + i0));
        const float be = sBeta[r];
        f32x4 xk, y, xq, qh;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i0 + j;
          const float g = sG[r * DK + i], gR = sG[16 * R * DK + i], gC = sG[(CH - 1) * DK + i];
          const float gread = p.literal ? (r > 0 ? sG[(r - 1) * DK + i] : 0.f) : g;
          xk[j] = be * kk[j] * __expf(gread - gR);
          y[j] = kk[j] * __expf(gR - g);
          xq[j] = qq[j] * __expf(g - gR);
          qh[j] = qq[j] * __expf(g);
          sKrT[i * LCH + r] = O::from(be * kk[j] * __expf(gread));
          sKdT[i * LCH + r] = O::from(kk[j] * __expf(gC - g));
        }
        *reinterpret_cast<frag*>(sK + r * LDK + i0) = O::cvt(xk);
        *reinterpret_cast<frag*>(sY + r * LDK + i0) = O::cvt(y);
        *reinterpret_cast<frag*>(sQ + r * LDK + i0) = O::cvt(xq);
        *reinterpret_cast<frag*>(sQh + r * LDK + i0) = O::cvt(qh);
      }
      __syncthreads();
    }

    // ---- (2) 16x16 blocks of A (strictly lower) and P (lower incl. diagonal) ------
    // Each wave forms the diagonal blocks of A it owns and inverts them in
    // registers; the 16 off-diagonal A blocks and P blocks are split evenly.
    auto block_product = [&](auto is_p, int R, int J) -> f32x4 {
      constexpr bool isP = decltype(is_p)::value;
      const T* rows = isP ? sQ : sK;
      const T* cols = RAW ? sK : sY;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const int c = 32 * kb + 4 * lg;
        frag a0 = O::ld(rows + (16 * R + lr) * LDK + c);
        frag a1 = O::ld(rows + (16 * R + lr) * LDK + c + 16);
        frag b0 = O::ld(cols + (16 * J + lr) * LDK + c);
        frag b1 = O::ld(cols + (16 * J + lr) * LDK + c + 16);
        if constexpr (GATE == GATE_CHANNEL) {
          if (R > J) {
            const float* m = sM + strict_pair(R, J) * DK + c;
            b0 = O::cvt(O::f32(b0) * *reinterpret_cast<const f32x4*>(m));
            b1 = O::cvt(O::f32(b1) * *reinterpret_cast<const f32x4*>(m + 16));
          }
        }
        acc = O::mma2(acc, a0, a1, b0, b1);
      }
      // decay and beta factors, then the causal mask
      const int j = 16 * J + lr;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int rr = 4 * lg + s, r = 16 * R + rr;
        float val = acc[s];
        if constexpr (GATE == GATE_SCALAR) val *= __expf((isP ? sGr[r] : sGrd[r]) - sGr[j]);
        if constexpr (RAW) {
          if (!isP) val *= sBr[r];
        }
        acc[s] = (R == J && (isP ? rr < lr : rr <= lr)) ? 0.f : val;
      }
      return acc;
    };
    for (int R = wave; R < 4; R += NW) {
      const f32x4 x = unit_lower_inverse(block_product(std::false_type{}, R, R), sScr + wave * 16 * L::LSC, lr, lg);
#pragma unroll
      for (int s = 0; s < 4; ++s) sXi[(16 * R + 4 * lg + s) * LXI + lr] = O::from(x[s]);
    }
    {
      // tasks [lo, hi) of the list: 6 strictly-lower A blocks, then 10 P blocks
      const int lo = 16 * wave / NW, hi = 16 * (wave + 1) / NW;
      for (int t = lo; t < (hi < 6 ? hi : 6); ++t) {
        const int R = 1 + (t >= 1) + (t >= 3), J = t - R * (R - 1) / 2;
        const f32x4 acc = block_product(std::false_type{}, R, J);
#pragma unroll
        for (int s = 0; s < 4; ++s) sA[(16 * R + 4 * lg + s) * LA + 16 * J + lr] = acc[s];
      }
      for (int t = (lo > 6 ? lo : 6); t < hi; ++t) {
        const int u = t - 6;
        const int R = (u >= 1) + (u >= 3) + (u >= 6), J = u - R * (R + 1) / 2;
        const f32x4 acc = block_product(std::true_type{}, R, J);
#pragma unroll
        for (int s = 0; s < 4; ++s) sP[(16 * R + 4 * lg + s) * LCH + 16 * J + lr] = O::from(acc[s]);
      }
    }
    __syncthreads();

    // ---- (3) W and U by block forward substitution (per wave, own columns) --------
    // out_R = X_RR (rhs_R - sum_{J<R} A_RJ out_J); the CBW channel blocks of W and
    // the wave's block of U advance together.
    constexpr int NB = CBW + 1;
    f32x4 outf[NB][4];
    frag outb[NB][4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      frag aR[3];
#pragma unroll
      for (int J = 0; J < R; ++J)
        aR[J] = O::cvt(-*reinterpret_cast<const f32x4*>(sA + (16 * R + lr) * LA + 16 * J + 4 * lg));
      const frag xi = O::ld(sXi + (16 * R + lr) * LXI + 4 * lg);
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        f32x4 acc;
        if (c < CBW) {
          const int ch = (wave * CBW + c) * 16 + lr;
          if constexpr (RAW) {
            acc = O::f32(O::ld(sKT + ch * LCH + 16 * R + 4 * lg));
#pragma unroll
            for (int s = 0; s < 4; ++s) acc[s] *= sEw[16 * R + 4 * lg + s];
          } else {
            acc = O::f32(O::ld(sKrT + ch * LCH + 16 * R + 4 * lg));
          }
        } else {
          acc = O::f32(O::ld(sVT + (16 * wave + lr) * LCH + 16 * R + 4 * lg));
#pragma unroll
          for (int s = 0; s < 4; ++s) acc[s] *= sBeta[16 * R + 4 * lg + s];
        }
        int J = 0;
#pragma unroll
        for (; J + 1 < R; J += 2) acc = O::mma2(acc, aR[J], aR[J + 1], outb[c][J], outb[c][J + 1]);
        if (J < R) acc = O::mma1(acc, aR[J], outb[c][J]);
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = O::mma1(z, xi, O::cvt(acc));
        outf[c][R] = z;
        outb[c][R] = O::cvt(z);
      }
    }
#pragma unroll
    for (int c = 0; c < CBW; ++c) {
      const int ch = (wave * CBW + c) * 16 + lr;
#pragma unroll
      for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int s = 0; s < 4; ++s) sW[(16 * R + 4 * lg + s) * LDK + ch] = O::from(outf[c][R][s]);
    }
    __syncthreads();

    // ---- (4) state pass and output for this wave's 16 columns ---------------------
    frag Sb[DKT];
#pragma unroll
    for (int t = 0; t < DKT; ++t) Sb[t] = O::cvt(S[t]);
    frag Db[4], Ds[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {            // Delta = U - W S
      f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const T* wr = sW + (16 * R + lr) * LDK + 32 * kb + 4 * lg;
        ws = O::mma2(ws, O::ld(wr), O::ld(wr + 16), Sb[2 * kb], Sb[2 * kb + 1]);
      }
      const f32x4 d = outf[CBW][R] - ws;
      Db[R] = O::cvt(d);
      if constexpr (GATE == GATE_SCALAR) {
        f32x4 ds;
#pragma unroll
        for (int s = 0; s < 4; ++s) ds[s] = d[s] * sEd[16 * R + 4 * lg + s];
        Ds[R] = O::cvt(ds);
      } else {
        Ds[R] = Db[R];
      }
    }
    // O^T tile (rows = this wave's 16 columns, columns = 16 tokens):
    //   S^T (Q e^g)^T + Delta^T P^T; a lane ends up with 4 adjacent output columns.
    const T* qsrc = RAW ? sQ : sQh;
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      f32x4 oq = {0.f, 0.f, 0.f, 0.f}, op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const T* qr = qsrc + (16 * R + lr) * LDK + 32 * kb + 4 * lg;
        oq = O::mma2(oq, Sb[2 * kb], Sb[2 * kb + 1], O::ld(qr), O::ld(qr + 16));
      }
      const T* pr = sP + (16 * R + lr) * LCH + 4 * lg;
      int J = 0;
#pragma unroll
      for (; J + 1 <= R; J += 2) op = O::mma2(op, Db[J], Db[J + 1], O::ld(pr + 16 * J), O::ld(pr + 16 * (J + 1)));
      if (J <= R) op = O::mma1(op, Db[J], O::ld(pr + 16 * J));
      const int r = 16 * R + lr;
      f32x4 ov;
      if constexpr (GATE == GATE_SCALAR) ov = oq * sEo[r] + op; else ov = oq + op;
      if (r < nrows) {
        elem* dst = go + tok(t0 + r) * dv + col0 + 16 * wave + 4 * lg;
        if constexpr (IO == IO_BF16) {
          const uint32_t lo = uint32_t(f32_to_bf16_bits(ov[0])) | (uint32_t(f32_to_bf16_bits(ov[1])) << 16);
          const uint32_t hi = uint32_t(f32_to_bf16_bits(ov[2])) | (uint32_t(f32_to_bf16_bits(ov[3])) << 16);
          *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(ov[0], ov[1], ov[2], ov[3]);
        }
      }
    }
    // S' = diag(e^{g_63}) S + (K e^{g_63 - g})^T Delta
    const T* kdt = RAW ? sKT : sKdT;
#pragma unroll
    for (int t = 0; t < DKT; ++t) {
      f32x4 acc = S[t];
      if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[s] *= sGamC[16 * t + 4 * lg + s];
      } else if constexpr (GATE == GATE_SCALAR) {
        acc = acc * sGamR[0];
      }
      const T* kr = kdt + (16 * t + lr) * LCH + 4 * lg;
      acc = O::mma2(acc, O::ld(kr), O::ld(kr + 16), Ds[0], Ds[1]);
      acc = O::mma2(acc, O::ld(kr + 32), O::ld(kr + 48), Ds[2], Ds[3]);
      S[t] = acc;
    }
    __syncthreads();                          // LDS is rewritten by the next chunk
  }

  if (p.S_T) {
#pragma unroll
    for (int t = 0; t < DKT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) p.S_T[(bh * DK + 16 * t + 4 * lg + s) * dv + scol] = S[t][s];
  }
}

template <int IO, int GATE, int DK, int NW>
static hipError_t launch_chunk_t(const ChunkParams& p, hipStream_t stream) {
  const int n_tiles = p.d_v / (16 * NW);
  const int64_t nblk = p.B * p.H * n_tiles;
  hipLaunchKernelGGL((chunk_fwd_kernel<IO, GATE, DK, NW>), dim3(static_cast<unsigned>(nblk)), dim3(NW * 64), 0,
                     stream, p, n_tiles);
  return hipGetLastError();
}

template <int IO, int GATE, int DK>
static hipError_t launch_chunk_dk(const ChunkParams& p, hipStream_t stream) {
  if constexpr (IO == IO_F32 || GATE == GATE_CHANNEL) {
    return launch_chunk_t<IO, GATE, DK, 2>(p, stream);   // LDS budget: 32-column tiles
  } else {
    // Four waves (64 columns per workgroup) when that still gives at least one
    // workgroup per CU, otherwise two waves (32 columns) to fill the 256 CUs.
    const int64_t wg4 = p.B * p.H * (p.d_v / 64);
    if (wg4 >= 256) return launch_chunk_t<IO, GATE, DK, 4>(p, stream);
    return launch_chunk_t<IO, GATE, DK, 2>(p, stream);
  }
}

template <int IO, int GATE>
static hipError_t launch_chunk_g(const ChunkParams& p, hipStream_t stream) {
  if (p.d_k == 128) {
    if constexpr (IO == IO_F32) {
      return hipErrorInvalidValue;   // fp32 I/O: d_k = 64 only (LDS budget)
    } else {
      return launch_chunk_dk<IO, GATE, 128>(p, stream);
    }
  }
  if (p.d_k == 64) return launch_chunk_dk<IO, GATE, 64>(p, stream);
  return hipErrorInvalidValue;
}

template <int IO>
static hipError_t launch_chunk_io(const ChunkParams& p, hipStream_t stream) {
  switch (p.gate) {
    case GATE_NONE: return launch_chunk_g<IO, GATE_NONE>(p, stream);
    case GATE_SCALAR: return launch_chunk_g<IO, GATE_SCALAR>(p, stream);
    case GATE_CHANNEL: return launch_chunk_g<IO, GATE_CHANNEL>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd(const ChunkParams& p, hipStream_t stream) {
  if (p.B * p.H == 0) return hipSuccess;
  return p.io == IO_BF16 ? launch_chunk_io<IO_BF16>(p, stream) : launch_chunk_io<IO_F32>(p, stream);
}

}  // namespace gdr
