// Per-chunk transform of the gated delta rule on gfx950: everything about a
// chunk that does not depend on the state, for every (batch, head, chunk) at once.
//
// "Moonshot AI's New Attention Architecture: Key Innovations Explained", §3
// Hardware-Friendly Algorithm: inside a chunk, the delta-rule correction terms
// come from a unit lower triangular system whose strictly lower part is the
// beta-weighted, gate-decayed Gram matrix of the chunk's keys, and the output
// adds a causally masked product of queries and keys; neither depends on the
// state passed between chunks.  With g_r the inclusive running sum of log a over
// the chunk rows (§5 Practical Considerations: the gate in the log domain),
//     A = strict_lower( diag(beta) (K * e^{g_read}) (K * e^{-g})^T ),
//     T = (I + A)^{-1},
//     P = lower_incl( (Q * e^{g}) (K * e^{-g})^T ),
// where g_read = g when the decay precedes the erase and g_{r-1} when the erase
// reads the undecayed state; without a per-channel gate also the per-row
// factors beta, e^{g_read}, e^{g}, e^{g_63 - g}, e^{g_63}, g in fp32.
//
// Written per chunk (the workspace record): the ten non-zero 16x16 blocks of T,
// each transposed, so that the state pass reads T's rows with the LDS
// transpose load, and (per-channel gate, fp32 I/O) the ten blocks of P.  With
// bf16 I/O and no per-channel gate the state pass forms P itself from the q and
// k tiles it holds anyway, which saves reading q here and a round trip of P
// through memory.  With bf16 I/O and a per-channel gate the record also carries
// the state pass's decayed operands k e^{g_read}, q e^{g}, k e^{g_63 - g}, beta and
// the chunk's per-channel decay e^{g_63}: they are formed once per (sequence,
// head, chunk) here rather than once per d_v tile there.
//
// No gate / scalar gate (chunk_prep_reg_kernel): one wave per chunk, every
// operand in registers.  The Gram sums run over d_k, so k and q are loaded as
// 16-byte pieces straight into MFMA operand registers (A and B take the same
// channel order, which leaves each sum unchanged).  An accumulator tile of X
// stands for X as the B operand of a product and for X^T as the A operand, so:
// the blocks A_Rm are formed transposed (operands swapped), which is the A
// operand of the solve; the symmetric diagonal Gram block gives both
// orientations of A_RR, whose inverse D_R is a finite Neumann product in
// registers (both orientations again); then row block R of T follows by
// forward substitution,
//     T_RR = D_R,   T_RJ = -D_R sum_{J <= m < R} A_Rm T_mJ,
// with T blocks kept as B operands.  P blocks (fp32 I/O) are formed transposed
// too, which is the layout of P's rows.  Everything is stored from the
// accumulators, four elements per lane, one whole 16x16 block per instruction;
// no LDS is used beyond 768 bytes of per-row factors.
//
// Per-channel gate (chunk_prep_chan_kernel for bf16 I/O, chunk_prep_lds_kernel
// for fp32 I/O): the decay sits inside the d_k contraction, so decayed operands
// are built in LDS by a four-wave workgroup per chunk; the factor e^{g_r - g_j} is split at the first row of each 16-row
// block (e^{g_r - g_16R} on the row operand, e^{g_16J - g_j} on the column
// operand, e^{g_16R - g_16J} on the column operand of blocks below the
// diagonal), so no operand carries more than 15 tokens of decay.  Wave R
// inverts I + A_RR (Neumann product on fp32 MFMA), the blocks below the diagonal
// are shared out, and wave J walks down block column J of T.
#include <type_traits>

#include "chunk_common.h"
#include "launchers.h"

namespace gdr {

template <int IO, int GATE, int DK>
struct PrepLayout {
  typedef typename Op<IO>::T T;
  static constexpr bool RAW = GATE != GATE_CHANNEL;
  static constexpr int PAD = Op<IO>::PAD;
  static constexpr int LDK = DK + PAD;
  static constexpr int LCH = CH + PAD;
  static constexpr int LSC = 20;
  static constexpr int NSEG = 256 / DK;                  // row segments of the per-channel scan
  static constexpr size_t RM = size_t(CH) * LDK * sizeof(T);
  static constexpr size_t MM = size_t(CH) * LCH * sizeof(T);
  static constexpr size_t OFF_K = 0;                      // raw k; per-channel: beta k e^{g_read - g_16R}
  static constexpr size_t OFF_Q = OFF_K + RM;             // raw q; per-channel: q e^{g - g_16R}
  static constexpr size_t OFF_A = OFF_Q + RM;             // A, blocks below the diagonal
  static constexpr size_t OFF_T = OFF_A + MM;             // result tiles
  static constexpr size_t OFF_P = OFF_T + MM;
  static constexpr size_t OFF_SC = OFF_P + MM;            // per-wave 16x16 fp32 scratch
  static constexpr size_t OFF_X = OFF_SC + 4 * 16 * LSC * 4;
  // no gate / scalar gate: beta, g, g_read
  static constexpr size_t R_TOTAL = OFF_X + 3 * CH * 4;
  // per-channel gate
  static constexpr size_t C_Y = OFF_X;                    // column operand k e^{g_16J - g}
  static constexpr size_t C_G = C_Y + RM;                 // g [64][DK] fp32
  static constexpr size_t C_BETA = C_G + size_t(CH) * DK * 4;
  static constexpr size_t C_M = C_BETA + CH * 4;          // e^{g_16R - g_16J}, 6 block pairs
  static constexpr size_t C_TOT = C_M + 6 * DK * 4;
  static constexpr size_t C_TOTAL = C_TOT + NSEG * DK * 4;
  static constexpr size_t TOTAL = RAW ? R_TOTAL : C_TOTAL;
};

template <int IO, int GATE, int DK>
__global__ __launch_bounds__(256) void chunk_prep_lds_kernel(ChunkParams p) {
  typedef Op<IO> O;
  typedef typename O::T T;
  typedef typename Io<IO>::elem elem;
  typedef PrepLayout<IO, GATE, DK> L;
  constexpr bool RAW = L::RAW;
  constexpr int NT = 256;
  constexpr int LDK = L::LDK, LCH = L::LCH;
  constexpr int ESZ = int(sizeof(elem));
  typedef WsRec<ESZ> W;
  constexpr int EPV = 16 / ESZ;                 // elements per 16-byte piece
  constexpr int KROW = DK / EPV;
  constexpr int KV = CH * KROW / NT;            // 16-byte pieces of the k (q) tile per thread
  static_assert(KV * NT == CH * KROW, "tile pieces must split evenly");
  static_assert(L::TOTAL <= 163840, "LDS budget");

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  T* sK = reinterpret_cast<T*>(smem + L::OFF_K);
  T* sQ = reinterpret_cast<T*>(smem + L::OFF_Q);
  T* sA = reinterpret_cast<T*>(smem + L::OFF_A);
  T* sT = reinterpret_cast<T*>(smem + L::OFF_T);
  T* sP = reinterpret_cast<T*>(smem + L::OFF_P);
  float* sScr = reinterpret_cast<float*>(smem + L::OFF_SC);
  float* sBr = reinterpret_cast<float*>(smem + L::OFF_X);
  float* sGr = sBr + CH;
  float* sGrd = sBr + 2 * CH;
  T* sY = reinterpret_cast<T*>(smem + L::C_Y);
  float* sG = reinterpret_cast<float*>(smem + L::C_G);
  float* sBc = reinterpret_cast<float*>(smem + L::C_BETA);
  float* sM = reinterpret_cast<float*>(smem + L::C_M);
  float* sTot = reinterpret_cast<float*>(smem + L::C_TOT);

  // block order (batch or slot, chunk, head), head fastest (see chunk_prep_reg_kernel)
  int64_t bb, n, hh;
  if (!prep_task(p, blockIdx.x, bb, n, hh)) return;   // whole workgroup: no chunk for this slot
  const SeqSpan sq = seq_span(p, bb, hh);
  const int H = static_cast<int>(p.H);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  char* rec = static_cast<char*>(p.ws) + (sq.rec0 + n) * W::BYTES;
  static_assert(IO == IO_F32 || GATE != GATE_CHANNEL, "bf16 per-channel gate: chunk_prep_chan_kernel");

  // The chunk's rows through buffers whose range ends at the sequence's last
  // token: rows of a ragged last chunk read as zero.
  const int64_t t0 = n * CH;
  const int64_t row0 = (sq.t0 + t0) * p.H + hh;         // token row of (b, t0, h)
  const int64_t left = sq.len - t0;                      // >= 1
  const uint32_t span = static_cast<uint32_t>(((left < CH ? left : CH) - 1) * p.H + 1);
  const rsrc_t rk = make_rsrc(static_cast<const elem*>(p.k) + row0 * DK, span * DK * ESZ);
  const rsrc_t rq = make_rsrc(static_cast<const elem*>(p.q) + row0 * DK, span * DK * ESZ);
  const rsrc_t rb = make_rsrc(static_cast<const elem*>(p.beta) + row0, span * ESZ);
  const rsrc_t rl = make_rsrc(static_cast<const elem*>(p.log_a) + row0 * (GATE == GATE_CHANNEL ? DK : 1),
                              GATE == GATE_NONE ? 0u : span * (GATE == GATE_CHANNEL ? DK : 1) * ESZ);
  auto to_f32 = [&](uint32_t bits) -> float {
    if constexpr (IO == IO_BF16) return bf16_bits_to_f32(static_cast<uint16_t>(bits));
    else return __uint_as_float(bits);
  };
  auto load1 = [&](rsrc_t r, uint32_t off) -> float {
    if constexpr (IO == IO_BF16) return to_f32(buf_load2(r, off, 0));
    else return to_f32(buf_load4(r, off, 0));
  };

  // ---- chunk into LDS -------------------------------------------------------------
#pragma unroll
  for (int v = 0; v < KV; ++v) {
    const int seg = tid + v * NT, row = seg / KROW, c = (seg % KROW) * EPV;
    const uint32_t off = static_cast<uint32_t>((row * H * DK + c) * ESZ);
    *reinterpret_cast<u32x4*>(sK + row * LDK + c) = buf_load16(rk, off, 0);
    *reinterpret_cast<u32x4*>(sQ + row * LDK + c) = buf_load16(rq, off, 0);
    if constexpr (GATE == GATE_CHANNEL) {
      const u32x4 w4 = buf_load16(rl, off, 0);
#pragma unroll
      for (int j = 0; j < EPV; ++j) {
        const uint32_t w = w4[j * ESZ / 4];
        sG[row * DK + c + j] = to_f32(ESZ == 2 ? (w >> (16 * (j & 1))) & 0xffffu : w);
      }
    }
  }
  if constexpr (RAW) {
    if (wave == 0) {              // inclusive scan of the log-gate; per-row factors
      const uint32_t off = static_cast<uint32_t>(lane * H * ESZ);
      const float b = load1(rb, off);
      float g = 0.f, gread = 0.f;
      if constexpr (GATE == GATE_SCALAR) {
        g = load1(rl, off);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const float y = __shfl_up(g, d);
          if (lane >= d) g += y;
        }
        const float gprev = __shfl_up(g, 1);
        gread = p.literal ? (lane == 0 ? 0.f : gprev) : g;
      }
      const float gC = __shfl(g, 63);
      sBr[lane] = b;
      sGr[lane] = g;
      sGrd[lane] = gread;
      float* f = reinterpret_cast<float*>(rec + W::F_OFF);
      f[lane] = b;
      f[CH + lane] = __expf(gread);
      f[2 * CH + lane] = __expf(g);
      f[3 * CH + lane] = __expf(gC - g);
      f[4 * CH + lane] = __expf(gC);
      f[5 * CH + lane] = g;
    }
  } else {
    if (tid < CH) sBc[tid] = load1(rb, static_cast<uint32_t>(tid * H * ESZ));
  }
  __syncthreads();

  if constexpr (!RAW) {
    // inclusive scan of the gate down each key channel, in NSEG row segments
    constexpr int NSEG = L::NSEG, SEGL = CH / NSEG;
    {
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
      const int i = tid % DK, seg = tid / DK;
      float pre = 0.f;
      for (int s2 = 0; s2 < seg; ++s2) pre += sTot[s2 * DK + i];
      if (seg > 0)
        for (int r = seg * SEGL; r < (seg + 1) * SEGL; ++r) sG[r * DK + i] += pre;
    }
    __syncthreads();
    // decays past the split's range go to the generic kernel (see SPLIT_MAX)
    bool wide = false;
    for (int task = tid; task < CH * DK; task += NT) {
      const int r = task / DK, i = task % DK;
      wide |= sG[16 * (r >> 4) * DK + i] - sG[r * DK + i] > SPLIT_MAX;
      if (p.literal && (r & 15) == 0)
        wide |= (r > 0 ? sG[(r - 1) * DK + i] : 0.f) - sG[r * DK + i] > SPLIT_MAX;
    }
    wide = __syncthreads_or(wide);
    if (tid == 0) *reinterpret_cast<float*>(rec + rec_flag_off<ESZ>()) = wide ? 1.f : 0.f;
    if (wide) return;                           // uniform over the workgroup
    for (int i = tid; i < DK; i += NT) {
#pragma unroll
      for (int R = 1; R < 4; ++R)
#pragma unroll
        for (int J = 0; J < R; ++J)
          sM[strict_pair(R, J) * DK + i] = __expf(sG[16 * R * DK + i] - sG[16 * J * DK + i]);
    }
    // decayed operands; the row operands overwrite the raw tiles in place
    for (int task = tid; task < CH * (DK / 4); task += NT) {
      const int r = task / (DK / 4), i0 = (task % (DK / 4)) * 4, R = r >> 4;
      const f32x4 kk = O::f32(O::ld(sK + r * LDK + i0));
      const f32x4 qq = O::f32(O::ld(sQ + r * LDK + i0));
      const float be = sBc[r];
      f32x4 xk, xq, y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j;
        const float g = sG[r * DK + i], gR = sG[16 * R * DK + i];
        const float gread = p.literal ? (r > 0 ? sG[(r - 1) * DK + i] : 0.f) : g;
        xk[j] = be * kk[j] * __expf(gread - gR);
        xq[j] = qq[j] * __expf(g - gR);
        y[j] = kk[j] * __expf(gR - g);
      }
      *reinterpret_cast<typename O::frag*>(sK + r * LDK + i0) = O::cvt(xk);
      *reinterpret_cast<typename O::frag*>(sQ + r * LDK + i0) = O::cvt(xq);
      *reinterpret_cast<typename O::frag*>(sY + r * LDK + i0) = O::cvt(y);
    }
    __syncthreads();
  }

  // ---- 16x16 blocks of A (strictly lower) and P (lower incl. diagonal) ------------------
  auto block = [&](auto is_p, int R, int J) -> f32x4 {
    constexpr bool isP = decltype(is_p)::value;
    const T* rows = isP ? sQ : sK;
    const T* cols = RAW ? sK : sY;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      const int c = 32 * kb + 4 * lg;
      const auto a0 = O::ld(rows + (16 * R + lr) * LDK + c);
      const auto a1 = O::ld(rows + (16 * R + lr) * LDK + c + 16);
      auto b0 = O::ld(cols + (16 * J + lr) * LDK + c);
      auto b1 = O::ld(cols + (16 * J + lr) * LDK + c + 16);
      if constexpr (GATE == GATE_CHANNEL) {
        if (R > J) {
          const float* m = sM + strict_pair(R, J) * DK + c;
          b0 = O::cvt(O::f32(b0) * *reinterpret_cast<const f32x4*>(m));
          b1 = O::cvt(O::f32(b1) * *reinterpret_cast<const f32x4*>(m + 16));
        }
      }
      acc = O::mma2(acc, a0, a1, b0, b1);
    }
    const int j = 16 * J + lr;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int rr = 4 * lg + s, r = 16 * R + rr;
      float val = acc[s];
      if constexpr (GATE == GATE_SCALAR) val *= __expf((isP ? sGr[r] : sGrd[r]) - sGr[j]);
      if constexpr (RAW && !isP) val *= sBr[r];
      acc[s] = (R == J && (isP ? rr < lr : rr <= lr)) ? 0.f : val;
    }
    return acc;
  };

  // diagonal block of this wave: T_RR = (I + A_RR)^{-1}, stored transposed (sT holds T^T)
  const int R0 = wave;
  const f32x4 Dw = unit_lower_inverse(block(std::false_type{}, R0, R0), sScr + wave * 16 * L::LSC, lr, lg);
#pragma unroll
  for (int s = 0; s < 4; ++s) sT[(16 * R0 + lr) * LCH + 16 * R0 + 4 * lg + s] = O::from(Dw[s]);
  // the six blocks of A below the diagonal, (1,0) (2,0) (2,1) (3,0) (3,1) (3,2):
  // task t goes to wave 3 - t % 4, so the wave with the longest column solve gets fewest
#pragma unroll
  for (int t = 0; t < 6; ++t) {
    if (3 - (t & 3) != wave) continue;
    const int R = 1 + (t >= 1) + (t >= 3), J = t - R * (R - 1) / 2;
    const f32x4 acc = block(std::false_type{}, R, J);
#pragma unroll
    for (int s = 0; s < 4; ++s) sA[(16 * R + 4 * lg + s) * LCH + 16 * J + lr] = O::from(acc[s]);
  }
  __syncthreads();

  // ---- block column J = wave of T by forward substitution ------------------------------
  {
    const int J = wave;
    typename O::frag Tb[4];
    Tb[0] = Tb[1] = Tb[2] = Tb[3] = O::cvt(Dw);
#pragma unroll
    for (int R = 1; R < 4; ++R) {
      if (R <= J) continue;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 3; ++m)
        if (m >= J && m < R) acc = O::mma1(acc, O::ld(sA + (16 * R + lr) * LCH + 16 * m + 4 * lg), Tb[m]);
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      z = O::mma1(z, O::ld_tr(sT, LCH, 16 * R, 16 * R, lr, lg), O::cvt(acc));   // rows of D_R from T^T
      z = -z;
      Tb[R] = O::cvt(z);
#pragma unroll
      for (int s = 0; s < 4; ++s) sT[(16 * J + lr) * LCH + 16 * R + 4 * lg + s] = O::from(z[s]);
    }
  }
  // ---- P blocks (0,0) (1,0) (1,1) (2,0) ... (3,3): wave w takes w + 1 of them ------------
  {
    const int first = 10 - (wave + 1) * (wave + 2) / 2;
    for (int u = first; u < first + wave + 1; ++u) {
      const int R = (u >= 1) + (u >= 3) + (u >= 6), J = u - R * (R + 1) / 2;
      const f32x4 acc = block(std::true_type{}, R, J);
#pragma unroll
      for (int s = 0; s < 4; ++s) sP[(16 * R + 4 * lg + s) * LCH + 16 * J + lr] = O::from(acc[s]);
    }
  }
  __syncthreads();

  // ---- the ten blocks of T (transposed) and of P to the workspace record -----------------
  constexpr int PPB = W::BLK * ESZ / 16;         // 16-byte pieces per block
  constexpr int PPR = PPB / 16;                  // pieces per block row
  for (int pc = tid; pc < 10 * PPB; pc += NT) {
    int R, J;
    tri_block(pc / PPB, R, J);
    const int a = (pc % PPB) / PPR, b0 = (pc % PPR) * EPV;
    *reinterpret_cast<u32x4*>(rec + W::T_OFF + pc * 16) =
        *reinterpret_cast<const u32x4*>(sT + (16 * J + a) * LCH + 16 * R + b0);
    *reinterpret_cast<u32x4*>(rec + W::P_OFF + pc * 16) =
        *reinterpret_cast<const u32x4*>(sP + (16 * R + a) * LCH + 16 * J + b0);
  }
}

// ---------------------------------------------------------------------------------
// Per-channel gate, bf16 I/O: one 256-thread workgroup per (sequence, head, chunk).
//
// Thread (cq, sg) owns channels 4cq..4cq+3 of the SL rows of segment sg.  It loads
// its pieces of k, q and log a straight into registers (for each row the
// threads of a segment read one contiguous stretch), runs the inclusive scan of
// the gate down its rows in registers, and takes the totals of the segments
// above it from LDS.  With g_16R the gate at the first row of the thread's
// 16-row block, every factor it needs comes from three exponentials per element:
//     a = e^{g - g_16R} <= 1,  b = e^{g_16R - g},  d = e^{g_63 - g} <= 1,
// and e^{g_16R} once per channel: the split operands of the Gram and score blocks
// (beta k e^{g_read - g_16R}, q a, k b) go to LDS, the state pass's operands
// (k e^{g_read}, q e^{g}, k d) to the workspace record.  Then, as in
// chunk_prep_lds_kernel, wave R inverts I + A_RR (fp32 MFMA), the blocks of A
// below the diagonal are shared out and wave J walks down block column J of T;
// the blocks of P are formed transposed and stored from the accumulators.  78 KB
// of LDS: two workgroups per CU overlap each other's loads and barriers.
// ---------------------------------------------------------------------------------
template <int DK>
struct ChanLayout {
  static constexpr int LDK = DK + 4;                      // b64 row reads (row 2 mod 8 dwords)
  static constexpr int LCH = CH + 8;                      // 16-byte aligned rows (T^T copied out in pieces)
  static constexpr int LSC = 20;
  static constexpr int NQ = DK / 4;                       // channel quads
  static constexpr int NSG = 256 / NQ;                    // row segments
  static constexpr int SL = CH / NSG;                     // rows per segment (8 or 4: inside one 16-row block)
  static constexpr size_t RM = size_t(CH) * LDK * 2;
  static constexpr size_t MM = size_t(CH) * LCH * 2;
  static constexpr size_t OFF_K = 0;                      // beta k e^{g_read - g_16R}
  static constexpr size_t OFF_Q = OFF_K + RM;             // q e^{g - g_16R}
  static constexpr size_t OFF_Y = OFF_Q + RM;             // k e^{g_16J - g}
  static constexpr size_t OFF_A = OFF_Y + RM;             // A below the diagonal; first the segment totals
  static constexpr size_t OFF_T = OFF_A + MM;             // T^T
  static constexpr size_t OFF_SC = OFF_T + MM;            // per-wave 16x16 fp32 scratch
  static constexpr size_t OFF_GB = OFF_SC + 4 * 16 * LSC * 4;   // g at rows 0, 16, 32, 48
  static constexpr size_t OFF_M = OFF_GB + 4 * DK * 4;    // e^{g_16R - g_16J}, 6 block pairs
  static constexpr size_t TOTAL = OFF_M + 6 * DK * 4;
  static_assert(NSG * SL == CH && 16 % SL == 0, "segments inside 16-row blocks");
  static_assert(size_t(NSG) * DK * 4 <= MM, "segment totals fit in the A region");
};

template <int DK>
__global__ __launch_bounds__(256, 2) void chunk_prep_chan_kernel(ChunkParams p) {
  typedef Op<IO_BF16> O;
  typedef __bf16 T;
  typedef uint16_t elem;
  typedef ChanLayout<DK> L;
  typedef WsRec<2> W;
  constexpr int NT = 256, ESZ = 2, EPV = 8;
  constexpr int LDK = L::LDK, LCH = L::LCH, NQ = L::NQ, NSG = L::NSG, SL = L::SL;
  static_assert(L::TOTAL <= 81920, "two workgroups per CU");

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  T* sK = reinterpret_cast<T*>(smem + L::OFF_K);
  T* sQ = reinterpret_cast<T*>(smem + L::OFF_Q);
  T* sY = reinterpret_cast<T*>(smem + L::OFF_Y);
  T* sA = reinterpret_cast<T*>(smem + L::OFF_A);
  float* sTot = reinterpret_cast<float*>(smem + L::OFF_A);
  T* sT = reinterpret_cast<T*>(smem + L::OFF_T);
  float* sScr = reinterpret_cast<float*>(smem + L::OFF_SC);
  float* sGb = reinterpret_cast<float*>(smem + L::OFF_GB);
  float* sM = reinterpret_cast<float*>(smem + L::OFF_M);

  // block order (batch or slot, chunk, head), head fastest (see chunk_prep_reg_kernel)
  int64_t bb, n, hh;
  if (!prep_task(p, blockIdx.x, bb, n, hh)) return;   // whole workgroup: no chunk for this slot
  const SeqSpan sq = seq_span(p, bb, hh);
  const int H = static_cast<int>(p.H);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  char* rec = static_cast<char*>(p.ws) + (sq.rec0 + n) * rec_bytes(IO_BF16, GATE_CHANNEL, DK);

  // the chunk's rows; rows of a ragged last chunk read as zero (no decay, no update)
  const int64_t t0 = n * CH;
  const int64_t row0 = (sq.t0 + t0) * p.H + hh;
  const int64_t left = sq.len - t0;
  const uint32_t span = static_cast<uint32_t>(((left < CH ? left : CH) - 1) * p.H + 1);
  const rsrc_t rk = make_rsrc(static_cast<const elem*>(p.k) + row0 * DK, span * DK * ESZ);
  const rsrc_t rq = make_rsrc(static_cast<const elem*>(p.q) + row0 * DK, span * DK * ESZ);
  const rsrc_t rl = make_rsrc(static_cast<const elem*>(p.log_a) + row0 * DK, span * DK * ESZ);
  const rsrc_t rb = make_rsrc(static_cast<const elem*>(p.beta) + row0, span * ESZ);

  const int cq = tid % NQ, sg = tid / NQ, c0 = 4 * cq, r0 = sg * SL, R = r0 / 16;
  u32x2 kr[SL], qr[SL], la[SL], kwr[SL];
  float be[SL];
#pragma unroll
  for (int j = 0; j < SL; ++j) {
    const uint32_t off = static_cast<uint32_t>(((r0 + j) * H * DK + c0) * ESZ);
    kr[j] = buf_load8(rk, off, 0);
    qr[j] = buf_load8(rq, off, 0);
    la[j] = buf_load8(rl, off, 0);
    be[j] = bf16_bits_to_f32(buf_load2(rb, static_cast<uint32_t>((r0 + j) * H * ESZ), 0));
  }
  // With a write key ("OSDN: Improving Delta Rule with Provable Online
  // Preconditioning in Linear Attention", §2.1) the column operand of the Gram and
  // score blocks and the state pass's update operand take kw; the rows of A and the
  // residual's operand keep k.
  if (p.kw) {
    const rsrc_t rkw = make_rsrc(static_cast<const elem*>(p.kw) + row0 * DK, span * DK * ESZ);
#pragma unroll
    for (int j = 0; j < SL; ++j) kwr[j] = buf_load8(rkw, static_cast<uint32_t>(((r0 + j) * H * DK + c0) * ESZ), 0);
  } else {
#pragma unroll
    for (int j = 0; j < SL; ++j) kwr[j] = kr[j];
  }
  auto el = [](u32x2 w, int c) -> float {       // element c of four packed bf16
    const uint32_t x = w[c >> 1];
    return __uint_as_float((c & 1) ? (x & 0xffff0000u) : (x << 16));
  };

  // inclusive scan of the gate down each channel: this segment in registers ...
  float g[SL][4];
  f32x4 run = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < SL; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      run[c] += el(la[j], c);
      g[j][c] = run[c];
    }
  *reinterpret_cast<f32x4*>(sTot + sg * DK + c0) = run;
  __syncthreads();
  // ... plus the totals of the segments above
  f32x4 pre = {0.f, 0.f, 0.f, 0.f};
  for (int s2 = 0; s2 < sg; ++s2) pre += *reinterpret_cast<const f32x4*>(sTot + s2 * DK + c0);
#pragma unroll
  for (int j = 0; j < SL; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) g[j][c] += pre[c];
  if (r0 % 16 == 0) *reinterpret_cast<f32x4*>(sGb + R * DK + c0) = f32x4{g[0][0], g[0][1], g[0][2], g[0][3]};
  __syncthreads();                              // g at the block starts in place; totals no longer read

  for (int i = tid; i < DK; i += NT) {
#pragma unroll
    for (int Rm = 1; Rm < 4; ++Rm)
#pragma unroll
      for (int J = 0; J < Rm; ++J) sM[strict_pair(Rm, J) * DK + i] = __expf(sGb[Rm * DK + i] - sGb[J * DK + i]);
  }
  const f32x4 gR = *reinterpret_cast<const f32x4*>(sGb + R * DK + c0);
  f32x4 eR, eprev;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    eR[c] = __expf(gR[c]);                      // e^{g_16R}
    eprev[c] = __expf(pre[c] - gR[c]);          // literal form, first row: e^{g_{r0-1} - g_16R}
  }
  // g_63 of each channel: the bottom segment holds it and shares it through the
  // segment-total region (nobody reads the totals after the last barrier)
  if (sg == NSG - 1)
    *reinterpret_cast<f32x4*>(sTot + c0) = f32x4{g[SL - 1][0], g[SL - 1][1], g[SL - 1][2], g[SL - 1][3]};
  __syncthreads();
  const f32x4 g63 = *reinterpret_cast<const f32x4*>(sTot + c0);
  float* f = reinterpret_cast<float*>(rec + W::F_OFF);
  if (sg == 0) *reinterpret_cast<f32x4*>(f + CH + c0) =
      f32x4{__expf(g63[0]), __expf(g63[1]), __expf(g63[2]), __expf(g63[3])};   // e^{g_63} per channel
  if (cq == 0)
#pragma unroll
    for (int j = 0; j < SL; ++j) f[r0 + j] = be[j];                                  // beta

  // operands
  f32x4 aprev = eprev;                          // e^{g_{r-1} - g_16R} of the previous row
#pragma unroll
  for (int j = 0; j < SL; ++j) {
    const int r = r0 + j;
    f32x4 xk, xq, y, sk, sq, sd;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float kk = el(kr[j], c), qq = el(qr[j], c), kwv = el(kwr[j], c);
      const float a = __expf(g[j][c] - gR[c]);
      const float ar = p.literal ? aprev[c] : a;             // e^{g_read - g_16R}
      aprev[c] = a;
      xk[c] = be[j] * kk * ar;
      xq[c] = qq * a;
      y[c] = kwv * __expf(gR[c] - g[j][c]);
      sk[c] = kk * ar * eR[c];
      sq[c] = qq * a * eR[c];
      sd[c] = kwv * __expf(g63[c] - g[j][c]);
    }
    *reinterpret_cast<bf16x4*>(sK + r * LDK + c0) = O::cvt(xk);
    *reinterpret_cast<bf16x4*>(sQ + r * LDK + c0) = O::cvt(xq);
    *reinterpret_cast<bf16x4*>(sY + r * LDK + c0) = O::cvt(y);
    char* x = rec + W::X_OFF + (r * DK + c0) * ESZ;
    *reinterpret_cast<u32x2*>(x) = __builtin_bit_cast(u32x2, to_bf16x4(sk));
    *reinterpret_cast<u32x2*>(x + CH * DK * ESZ) = __builtin_bit_cast(u32x2, to_bf16x4(sq));
    *reinterpret_cast<u32x2*>(x + 2 * CH * DK * ESZ) = __builtin_bit_cast(u32x2, to_bf16x4(sd));
  }
  // A decay beyond e^-SPLIT_MAX inside this thread's rows of the block (the column
  // factor e^{g_16R - g}), or, literal form, on the row before the block (the first
  // row's read factor e^{g_{16R-1} - g_16R}), leaves the chunk to the generic kernel.
  // The state pass's operands above carry factors <= 1 and stand as written.
  bool wide = false;
#pragma unroll
  for (int j = 0; j < SL; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) wide |= gR[c] - g[j][c] > SPLIT_MAX;
  if (p.literal && r0 % 16 == 0)
#pragma unroll
    for (int c = 0; c < 4; ++c) wide |= pre[c] - gR[c] > SPLIT_MAX;
  wide = __syncthreads_or(wide);
  if (tid == 0) *reinterpret_cast<float*>(rec + rec_flag_off<2>()) = wide ? 1.f : 0.f;
  if (wide) return;                             // uniform over the workgroup

  // ---- 16x16 blocks: rows (R) of sK or sQ against rows (J) of sY, the column operand
  // carrying e^{g_16R - g_16J} below the diagonal.  With `tr` the product is formed
  // transposed (operands swapped): acc[s] is element (16R + lr, 16J + 4lg + s)
  // instead of (16R + 4lg + s, 16J + lr).
  auto block = [&](const T* rows, int Rb, int J, bool tr) -> f32x4 {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      const int c = 32 * kb + 4 * lg;
      const bf16x4 a0 = O::ld(rows + (16 * Rb + lr) * LDK + c), a1 = O::ld(rows + (16 * Rb + lr) * LDK + c + 16);
      bf16x4 b0 = O::ld(sY + (16 * J + lr) * LDK + c), b1 = O::ld(sY + (16 * J + lr) * LDK + c + 16);
      if (Rb > J) {
        const float* m = sM + strict_pair(Rb, J) * DK + c;
        b0 = O::cvt(O::f32(b0) * *reinterpret_cast<const f32x4*>(m));
        b1 = O::cvt(O::f32(b1) * *reinterpret_cast<const f32x4*>(m + 16));
      }
      acc = tr ? O::mma2(acc, b0, b1, a0, a1) : O::mma2(acc, a0, a1, b0, b1);
    }
    return acc;
  };
  auto a_block = [&](int Rb, int J) -> f32x4 {  // strictly lower part of A
    f32x4 acc = block(sK, Rb, J, false);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (Rb == J && 4 * lg + s <= lr) acc[s] = 0.f;
    return acc;
  };

  // diagonal block of this wave: T_RR = (I + A_RR)^{-1}, stored transposed (sT holds T^T)
  const int R0 = wave;
  const f32x4 Dw = unit_lower_inverse(a_block(R0, R0), sScr + wave * 16 * L::LSC, lr, lg);
#pragma unroll
  for (int s = 0; s < 4; ++s) sT[(16 * R0 + lr) * LCH + 16 * R0 + 4 * lg + s] = O::from(Dw[s]);
  // the six blocks of A below the diagonal: task t goes to wave 3 - t % 4, so the
  // wave with the longest column solve gets fewest
#pragma unroll
  for (int t = 0; t < 6; ++t) {
    if (3 - (t & 3) != wave) continue;
    const int Rb = 1 + (t >= 1) + (t >= 3), J = t - Rb * (Rb - 1) / 2;
    const f32x4 acc = a_block(Rb, J);
#pragma unroll
    for (int s = 0; s < 4; ++s) sA[(16 * Rb + 4 * lg + s) * LCH + 16 * J + lr] = O::from(acc[s]);
  }
  __syncthreads();

  // ---- block column J = wave of T by forward substitution ------------------------------
  {
    const int J = wave;
    bf16x4 Tb[4];
    Tb[0] = Tb[1] = Tb[2] = Tb[3] = O::cvt(Dw);
#pragma unroll
    for (int Rb = 1; Rb < 4; ++Rb) {
      if (Rb <= J) continue;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 3; ++m)
        if (m >= J && m < Rb) acc = O::mma1(acc, O::ld(sA + (16 * Rb + lr) * LCH + 16 * m + 4 * lg), Tb[m]);
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      z = O::mma1(z, O::ld_tr(sT, LCH, 16 * Rb, 16 * Rb, lr, lg), O::cvt(acc));   // rows of D_R from T^T
      z = -z;
      Tb[Rb] = O::cvt(z);
#pragma unroll
      for (int s = 0; s < 4; ++s) sT[(16 * J + lr) * LCH + 16 * Rb + 4 * lg + s] = O::from(z[s]);
    }
  }
  // ---- P blocks (0,0) (1,0) (1,1) (2,0) ... (3,3): wave w takes w + 1 of them, formed
  // transposed (four adjacent columns per lane) and stored straight to the record
  {
    const int first = 10 - (wave + 1) * (wave + 2) / 2;
    for (int u = first; u < first + wave + 1; ++u) {
      int Rb, J;
      tri_block(u, Rb, J);
      f32x4 acc = block(sQ, Rb, J, true);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (Rb == J && 4 * lg + s > lr) acc[s] = 0.f;
      *reinterpret_cast<u32x2*>(rec + W::P_OFF + W::at(Rb, J, lr, 4 * lg)) = __builtin_bit_cast(u32x2, to_bf16x4(acc));
    }
  }
  __syncthreads();

  // ---- the ten blocks of T (transposed) to the record -----------------------------------
  constexpr int PPB = W::BLK * ESZ / 16, PPR = PPB / 16;
  for (int pc = tid; pc < 10 * PPB; pc += NT) {
    int Rb, J;
    tri_block(pc / PPB, Rb, J);
    const int a = (pc % PPB) / PPR, b0 = (pc % PPR) * EPV;
    *reinterpret_cast<u32x4*>(rec + W::T_OFF + pc * 16) =
        *reinterpret_cast<const u32x4*>(sT + (16 * J + a) * LCH + 16 * Rb + b0);
  }
}

// ---------------------------------------------------------------------------------
// Per-channel gate, chunks whose decay inside a 16-row block exceeds the split's
// range (marked by the transform, see SPLIT_MAX): their T and P blocks are formed
// again in fp32 with every decay taken as one exponential of a non-positive
// exponent,
//     A_rj = beta_r sum_c k_rc k_jc e^{g_read,rc - g_jc}   (j < r),
//     P_rj = sum_c q_rc k_jc e^{g_rc - g_jc}                (j <= r),
//     T    = (I + A)^{-1}, by forward substitution, one column per thread.
// One workgroup covers 256 transform tasks: each thread reads one task's mark, the
// marked ones are listed in LDS and the workgroup forms them one after another.
// The rest of the record (the state pass's operands and factors, all carrying
// factors <= 1) stands as the transform wrote it.
// ---------------------------------------------------------------------------------
template <int DK, int ESZ>
struct GenLayout {
  static constexpr int LK = DK + 1;                  // odd strides: rows r and j of one column sit in different banks
  static constexpr int LT = CH + 1;
  static constexpr size_t KT = (size_t(CH) * LK * ESZ + 15) / 16 * 16;   // one [64][LK] tile in the I/O dtype
  static constexpr size_t OFF_K = 0;                                // k
  static constexpr size_t OFF_Q = OFF_K + KT;                       // q
  static constexpr size_t OFF_KW = OFF_Q + KT;                      // the write key (or k again)
  static constexpr size_t OFF_G = OFF_KW + KT;                      // [65][LK] fp32: row 0 zero, row r + 1 = g_r
  static constexpr size_t OFF_A = OFF_G + size_t(CH + 1) * LK * 4;  // A [64][LT] fp32
  static constexpr size_t OFF_T = OFF_A + size_t(CH) * LT * 4;      // T [64][LT] fp32
  static constexpr size_t OFF_B = OFF_T + size_t(CH) * LT * 4;      // beta [64]
  static constexpr size_t TOTAL = OFF_B + CH * 4;
};

template <int IO, int DK>
__global__ __launch_bounds__(256) void chunk_prep_generic_kernel(ChunkParams p, int64_t ntasks) {
  typedef typename Io<IO>::elem elem;
  constexpr int ESZ = int(sizeof(elem));
  typedef WsRec<ESZ> W;
  typedef GenLayout<DK, ESZ> L;
  constexpr int NT = 256, LK = L::LK, LT = L::LT;
  constexpr uint32_t RB = rec_bytes(IO, GATE_CHANNEL, DK);
  static_assert(L::TOTAL <= 163840, "LDS budget");

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  __shared__ int s_list[NT];
  __shared__ int s_n;
  elem* sK = reinterpret_cast<elem*>(smem + L::OFF_K);
  elem* sQ = reinterpret_cast<elem*>(smem + L::OFF_Q);
  elem* sKW = reinterpret_cast<elem*>(smem + L::OFF_KW);
  float* sG = reinterpret_cast<float*>(smem + L::OFF_G);
  float* sA = reinterpret_cast<float*>(smem + L::OFF_A);
  float* sT = reinterpret_cast<float*>(smem + L::OFF_T);
  float* sB = reinterpret_cast<float*>(smem + L::OFF_B);
  const int tid = threadIdx.x;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * NT;

  if (tid == 0) s_n = 0;
  __syncthreads();
  {
    const int64_t task = base + tid;
    int64_t rec;
    if (task < ntasks && task_record(p, task, rec)) {
      const float mark = *reinterpret_cast<const float*>(static_cast<const char*>(p.ws) + rec * RB + rec_flag_off<ESZ>());
      if (mark != 0.f) s_list[atomicAdd(&s_n, 1)] = tid;
    }
  }
  __syncthreads();
  const int nmarked = s_n;

  auto load1 = [&](rsrc_t r, uint32_t off) -> float {
    if constexpr (IO == IO_BF16) return bf16_bits_to_f32(buf_load2(r, off, 0));
    else return __uint_as_float(buf_load4(r, off, 0));
  };
  auto loade = [&](rsrc_t r, uint32_t off) -> elem {
    if constexpr (IO == IO_BF16) return buf_load2(r, off, 0);
    else return __uint_as_float(buf_load4(r, off, 0));
  };
  auto f = [&](elem x) -> float {
    if constexpr (IO == IO_BF16) return bf16_bits_to_f32(x);
    else return x;
  };
  for (int m = 0; m < nmarked; ++m) {
    const int64_t task = uni64(base + s_list[m]);
    int64_t bb, n, hh;
    prep_task(p, task, bb, n, hh);              // a listed task has a chunk
    const SeqSpan sq = seq_span(p, bb, hh);
    const int H = static_cast<int>(p.H);
    char* rec = static_cast<char*>(p.ws) + (sq.rec0 + n) * RB;
    // the chunk's rows; rows past the end of the sequence read as zero
    const int64_t t0 = n * CH;
    const int64_t row0 = (sq.t0 + t0) * p.H + hh;
    const int64_t left = sq.len - t0;
    const uint32_t span = static_cast<uint32_t>(((left < CH ? left : CH) - 1) * p.H + 1);
    const rsrc_t rk = make_rsrc(static_cast<const elem*>(p.k) + row0 * DK, span * DK * ESZ);
    const rsrc_t rq = make_rsrc(static_cast<const elem*>(p.q) + row0 * DK, span * DK * ESZ);
    const rsrc_t rl = make_rsrc(static_cast<const elem*>(p.log_a) + row0 * DK, span * DK * ESZ);
    const rsrc_t rb = make_rsrc(static_cast<const elem*>(p.beta) + row0, span * ESZ);
    // the write key of "OSDN: Improving Delta Rule with Provable Online Preconditioning
    // in Linear Attention", §2.1 pairs with k in A and with q in P (columns j)
    const rsrc_t rkw = make_rsrc(static_cast<const elem*>(p.kw ? p.kw : p.k) + row0 * DK, span * DK * ESZ);

    __syncthreads();                            // the previous chunk's tiles are no longer read
    for (int e = tid; e < CH * DK; e += NT) {
      const int r = e / DK, c = e % DK;
      const uint32_t off = static_cast<uint32_t>((r * H * DK + c) * ESZ);
      sK[r * LK + c] = loade(rk, off);
      sQ[r * LK + c] = loade(rq, off);
      sKW[r * LK + c] = loade(rkw, off);
      sG[(r + 1) * LK + c] = load1(rl, off);
    }
    for (int c = tid; c < DK; c += NT) sG[c] = 0.f;
    if (tid < CH) sB[tid] = load1(rb, static_cast<uint32_t>(tid * H * ESZ));
    __syncthreads();
    for (int c = tid; c < DK; c += NT) {        // inclusive running sum down each channel
      float acc = 0.f;
      for (int r = 0; r < CH; ++r) {
        acc += sG[(r + 1) * LK + c];
        sG[(r + 1) * LK + c] = acc;
      }
    }
    __syncthreads();

    // one (r, j) pair, j <= r, per thread at a time
    for (int pr = tid; pr < CH * (CH + 1) / 2; pr += NT) {
      int r = static_cast<int>((sqrtf(8.f * pr + 1.f) - 1.f) * 0.5f);
      while (r * (r + 1) / 2 > pr) --r;
      while ((r + 1) * (r + 2) / 2 <= pr) ++r;
      const int j = pr - r * (r + 1) / 2;
      const elem* kr = sK + r * LK;
      const elem* kj = sKW + j * LK;            // column side: the write key (k without one)
      const elem* qr = sQ + r * LK;
      const float* gr = sG + (r + 1) * LK;
      const float* grd = sG + (p.literal ? r : r + 1) * LK;   // g_read: g_r, or g_{r-1} (g_{-1} = 0)
      const float* gj = sG + (j + 1) * LK;
      float a = 0.f, pv = 0.f;
      if (j < r) {
        for (int c = 0; c < DK; ++c) {
          a += f(kr[c]) * f(kj[c]) * __expf(grd[c] - gj[c]);
          pv += f(qr[c]) * f(kj[c]) * __expf(gr[c] - gj[c]);
        }
      } else {
        for (int c = 0; c < DK; ++c) pv += f(qr[c]) * f(kj[c]);
      }
      sA[r * LT + j] = j < r ? sB[r] * a : 0.f;
      const int R = r >> 4, J = j >> 4;
      Io<IO>::store(reinterpret_cast<elem*>(rec + W::P_OFF), W::at(R, J, r & 15, j & 15) / ESZ, pv);
      if (R == J && j < r)                      // the zero above the diagonal of a diagonal block
        Io<IO>::store(reinterpret_cast<elem*>(rec + W::P_OFF), W::at(R, J, j & 15, r & 15) / ESZ, 0.f);
    }
    __syncthreads();
    if (tid < CH) {                             // column j of T = (I + A)^{-1}
      const int j = tid;
      for (int i = 0; i < j; ++i) sT[i * LT + j] = 0.f;
      sT[j * LT + j] = 1.f;
      for (int i = j + 1; i < CH; ++i) {
        float s = 0.f;
        for (int m2 = j; m2 < i; ++m2) s += sA[i * LT + m2] * sT[m2 * LT + j];
        sT[i * LT + j] = -s;
      }
    }
    __syncthreads();
    // block (R, J) of the T region holds (T_RJ)^T: element (a, b) = T[16R + b][16J + a]
    for (int e = tid; e < 10 * 256; e += NT) {
      const int u = e >> 8, a = (e >> 4) & 15, b = e & 15;
      int R, J;
      tri_block(u, R, J);
      Io<IO>::store(reinterpret_cast<elem*>(rec + W::T_OFF), W::at(R, J, a, b) / ESZ,
                    sT[(16 * R + b) * LT + 16 * J + a]);
    }
  }
}

// ---------------------------------------------------------------------------------
// No gate / scalar gate: one wave per (sequence, head, chunk), operands in registers.
// ---------------------------------------------------------------------------------
template <int IO, int GATE, int DK>
__global__ __launch_bounds__(64) void chunk_prep_reg_kernel(ChunkParams p, int64_t ntasks) {
  typedef Op<IO> O;
  typedef typename O::frag frag;
  typedef typename Io<IO>::elem elem;
  constexpr int ESZ = int(sizeof(elem));
  typedef WsRec<ESZ> W;
  constexpr int EPV = 16 / ESZ;                 // elements per 16-byte piece
  constexpr int NSTEP = DK / (4 * EPV);         // products over d_k (four lane groups, one piece each)
  static_assert(GATE != GATE_CHANNEL, "per-channel gate uses chunk_prep_lds_kernel");
  static_assert(!gate_wkey(GATE) || IO == IO_BF16, "write key: bf16 I/O only");
  static_assert(NSTEP * 4 * EPV == DK, "d_k must split into pieces");

  // One wave per workgroup: a workgroup's registers and LDS are freed as soon as its
  // chunk is done, whatever its neighbours' loads are waiting on (measured 2-3 us
  // faster per call on the gated B8 H16 T8192 workload than four waves per workgroup).
  __shared__ __attribute__((aligned(16))) float sfac[3 * CH];   // beta, g, g_read
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  // Task order (batch or slot, chunk, head), head fastest: waves running side by
  // side read the whole token rows [t][H][d_k] of one chunk of one sequence together.
  const int64_t task = blockIdx.x;
  if (task >= ntasks) return;
  int64_t bb, n, hh;
  if (!prep_task(p, task, bb, n, hh)) return;   // a slot past the end of its sequence
  const SeqSpan sq = seq_span(p, bb, hh);
  const int H = static_cast<int>(p.H);
  char* rec = static_cast<char*>(p.ws) + (sq.rec0 + n) * rec_bytes(IO, GATE, DK);
  float* sB = sfac;
  float* sG = sB + CH;
  float* sGr = sB + 2 * CH;

  // The chunk's rows through buffers whose range ends at the sequence's last token.
  const int64_t t0 = n * CH;
  const int64_t row0 = (sq.t0 + t0) * p.H + hh;
  const int64_t left = sq.len - t0;
  const uint32_t span = static_cast<uint32_t>(((left < CH ? left : CH) - 1) * p.H + 1);
  const rsrc_t rk = make_rsrc(static_cast<const elem*>(p.k) + row0 * DK, span * DK * ESZ);
  const rsrc_t rq = make_rsrc(static_cast<const elem*>(p.q) + row0 * DK, span * DK * ESZ);
  const rsrc_t rb = make_rsrc(static_cast<const elem*>(p.beta) + row0, span * ESZ);
  const rsrc_t rl = make_rsrc(static_cast<const elem*>(p.log_a) + row0, gate_scalar(GATE) ? span * ESZ : 0u);
  auto load1 = [&](rsrc_t r, uint32_t off) -> float {
    if constexpr (IO == IO_BF16) return bf16_bits_to_f32(buf_load2(r, off, 0));
    else return __uint_as_float(buf_load4(r, off, 0));
  };
  // Write key (GATE_WKEY): the Gram matrix pairs the key of row r with the write
  // key of row j, A_rj = beta_r (k_r . kw_j), so kw takes the place of k on the
  // column side of every A block.
  constexpr bool WK = gate_wkey(GATE);
  const rsrc_t rkw = make_rsrc(static_cast<const elem*>(WK ? p.kw : p.k) + row0 * DK, span * DK * ESZ);
  // piece i of row block R: row 16R + lr, channels [(4i + lg) EPV, (4i + lg + 1) EPV)
  auto piece_off = [&](int R, int i) -> uint32_t {
    return static_cast<uint32_t>(((16 * R + lr) * H * DK + (4 * i + lg) * EPV) * ESZ);
  };
  u32x4 kf[4][NSTEP];
#pragma unroll
  for (int R = 0; R < 4; ++R)
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) kf[R][i] = buf_load16(rk, piece_off(R, i), 0);
  u32x4 kwf[WK ? 4 : 1][NSTEP];
  if constexpr (WK)
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
      for (int i = 0; i < NSTEP; ++i) kwf[R][i] = buf_load16(rkw, piece_off(R, i), 0);
  auto kcol = [&](int R) -> const u32x4* {       // column-side key pieces of row block R
    if constexpr (WK) return kwf[R];
    else return kf[R];
  };

  // ---- per-row gate factors (lane = row) ---------------------------------------------
  {
    const uint32_t off = static_cast<uint32_t>(lane * H * ESZ);
    const float b = load1(rb, off);
    float g = 0.f, gread = 0.f;
    if constexpr (gate_scalar(GATE)) {
      g = load1(rl, off);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(g, d);
        if (lane >= d) g += y;
      }
      const float gprev = __shfl_up(g, 1);
      gread = p.literal ? (lane == 0 ? 0.f : gprev) : g;
    }
    const float gC = __shfl(g, 63);
    sB[lane] = b;
    sG[lane] = g;
    sGr[lane] = gread;
    float* f = reinterpret_cast<float*>(rec + W::F_OFF);
    f[lane] = b;
    f[CH + lane] = __expf(gread);
    f[2 * CH + lane] = __expf(g);
    f[3 * CH + lane] = __expf(gC - g);
    f[4 * CH + lane] = __expf(gC);
    f[5 * CH + lane] = g;
  }
  wave_sync();

  auto gram = [&](const u32x4* a, const u32x4* b) -> f32x4 {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if constexpr (IO == IO_BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[i]),
                                                     acc, 0, 0, 0);
      } else {
        acc = mma_k16_f32(acc, __builtin_bit_cast(f32x4, a[i]), __builtin_bit_cast(f32x4, b[i]));
      }
    }
    return acc;
  };
  // four consecutive elements of a row of a record block
  auto store4 = [&](uint32_t off, f32x4 x) {
    char* d = rec + off;
    if constexpr (IO == IO_BF16) *reinterpret_cast<u32x2*>(d) = __builtin_bit_cast(u32x2, to_bf16x4(x));
    else *reinterpret_cast<u32x4*>(d) = __builtin_bit_cast(u32x4, x);
  };
  // element s of a transposed-product tile sits at row r = 16R + lr, column j = 16J + 4lg + s;
  // A factor: beta_r e^{g_read_r - g_j}
  auto a_factor = [&](f32x4 acc, int R, int J) -> f32x4 {
    const float br = sB[16 * R + lr], grr = sGr[16 * R + lr];
    const f32x4 gj = *reinterpret_cast<const f32x4*>(sG + 16 * J + 4 * lg);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float v = acc[s] * br;
      if constexpr (gate_scalar(GATE)) v *= __expf(grr - gj[s]);
      acc[s] = (R == J && lr <= 4 * lg + s) ? 0.f : v;
    }
    return acc;
  };

  constexpr bool WITH_P = IO == IO_F32;           // bf16: the state pass forms P itself
  frag Tb[4][4];                                  // Tb[R][J] = T_RJ as a B operand (J <= R)
#pragma unroll
  for (int R = 0; R < 4; ++R) {
    u32x4 qf[NSTEP];
    if constexpr (WITH_P) {
#pragma unroll
      for (int i = 0; i < NSTEP; ++i) qf[i] = buf_load16(rq, piece_off(R, i), 0);
    }

    // A_Rm (m < R) as A operands: transposed Gram blocks
    frag aRow[3];
#pragma unroll
    for (int m = 0; m < R; ++m) aRow[m] = O::cvt(a_factor(gram(kcol(m), kf[R]), R, m));
    // diagonal block, both orientations, and its inverse (without a write key the
    // Gram block is symmetric and one product serves both)
    const f32x4 G = gram(kcol(R), kf[R]);
    const f32x4 Nt = a_factor(G, R, R);         // accumulator tile of A_RR^T
    f32x4 N;                                       // accumulator tile of A_RR: row 16R+4lg+s, column 16R+lr
    {
      f32x4 G2 = G;
      if constexpr (WK) G2 = gram(kf[R], kcol(R));
      const f32x4 br = *reinterpret_cast<const f32x4*>(sB + 16 * R + 4 * lg);
      const f32x4 grr = *reinterpret_cast<const f32x4*>(sGr + 16 * R + 4 * lg);
      const float gj = sG[16 * R + lr];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float v = G2[s] * br[s];
        if constexpr (gate_scalar(GATE)) v *= __expf(grr[s] - gj);
        N[s] = (4 * lg + s > lr) ? v : 0.f;
      }
    }
    f32x4 D, Dt;
    unit_lower_inverse_pair<O>(N, Nt, D, Dt, lr, lg);
    Tb[R][R] = O::cvt(D);
    store4(W::T_OFF + W::at(R, R, lr, 4 * lg), D);         // (T_RR)^T
    const frag dA = O::cvt(Dt);                             // D_R as an A operand
#pragma unroll
    for (int J = 0; J < R; ++J) {
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = J; m < R; ++m) y = O::mma1(y, aRow[m], Tb[m][J]);
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
      t = O::mma1(t, dA, O::cvt(y));
      t = -t;
      Tb[R][J] = O::cvt(t);
      store4(W::T_OFF + W::at(R, J, lr, 4 * lg), t);       // (T_RJ)^T
    }

    // P row block R: transposed products give P's rows; factor e^{g_r - g_j}, mask r >= j
    if constexpr (!WITH_P) continue;
    const float gr = sG[16 * R + lr];
#pragma unroll
    for (int J = 0; J <= R; ++J) {
      f32x4 acc = gram(kf[J], qf);
      const f32x4 gj = *reinterpret_cast<const f32x4*>(sG + 16 * J + 4 * lg);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float v = acc[s];
        if constexpr (gate_scalar(GATE)) v *= __expf(gr - gj[s]);
        acc[s] = (J == R && lr < 4 * lg + s) ? 0.f : v;
      }
      store4(W::P_OFF + W::at(R, J, lr, 4 * lg), acc);
    }
  }
}

template <int IO, int GATE, int DK>
static hipError_t launch_prep_t(const ChunkParams& p, int64_t nchunks, hipStream_t stream) {
  const int64_t ntasks = p.cu ? p.H * p.nslots : p.B * p.H * nchunks;
  if constexpr (GATE == GATE_CHANNEL && IO == IO_BF16) {
    hipLaunchKernelGGL((chunk_prep_chan_kernel<DK>), dim3(static_cast<unsigned>(ntasks)), dim3(256), 0, stream, p);
  } else if constexpr (GATE == GATE_CHANNEL || (IO == IO_F32 && DK == 128)) {
    // fp32 at d_k = 128: the operands of a chunk do not fit a wave's registers, so
    // the four-wave kernel takes them through LDS
    hipLaunchKernelGGL((chunk_prep_lds_kernel<IO, GATE, DK>), dim3(static_cast<unsigned>(ntasks)), dim3(256), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((chunk_prep_reg_kernel<IO, GATE, DK>), dim3(static_cast<unsigned>(ntasks)), dim3(64), 0,
                       stream, p, ntasks);
  }
  if constexpr (GATE == GATE_CHANNEL) {
    // chunks whose decay leaves the split's range: T and P formed again
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_prep_generic_kernel<IO, DK>), dim3(static_cast<unsigned>((ntasks + 255) / 256)),
                       dim3(256), 0, stream, p, ntasks);
  }
  return hipGetLastError();
}

template <int IO, int GATE>
static hipError_t launch_prep_g(const ChunkParams& p, int64_t nchunks, hipStream_t stream) {
  if (p.d_k == 128) {
    if constexpr (IO == IO_F32 && GATE == GATE_CHANNEL) return hipErrorInvalidValue;   // LDS budget
    else return launch_prep_t<IO, GATE, 128>(p, nchunks, stream);
  }
  if (p.d_k == 64) return launch_prep_t<IO, GATE, 64>(p, nchunks, stream);
  return hipErrorInvalidValue;
}

template <int IO>
static hipError_t launch_prep_io(const ChunkParams& p, int64_t nchunks, hipStream_t stream) {
  if (p.kw) {
    if constexpr (IO == IO_BF16) {
      if (p.gate == GATE_NONE) return launch_prep_g<IO, GATE_WKEY>(p, nchunks, stream);
      if (p.gate == GATE_SCALAR) return launch_prep_g<IO, GATE_WKEY_SCALAR>(p, nchunks, stream);
      if (p.gate == GATE_CHANNEL) return launch_prep_g<IO, GATE_CHANNEL>(p, nchunks, stream);   // reads p.kw
      return hipErrorInvalidValue;
    }
    else return hipErrorInvalidValue;
  }
  switch (p.gate) {
    case GATE_NONE: return launch_prep_g<IO, GATE_NONE>(p, nchunks, stream);
    case GATE_SCALAR: return launch_prep_g<IO, GATE_SCALAR>(p, nchunks, stream);
    case GATE_CHANNEL: return launch_prep_g<IO, GATE_CHANNEL>(p, nchunks, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_prep(const ChunkParams& p, hipStream_t stream) {
  const int64_t nchunks = (p.T + CH - 1) / CH;
  if (p.B * p.H * nchunks == 0) return hipSuccess;
  return p.io == IO_BF16 ? launch_prep_io<IO_BF16>(p, nchunks, stream) : launch_prep_io<IO_F32>(p, nchunks, stream);
}

}  // namespace gdr
