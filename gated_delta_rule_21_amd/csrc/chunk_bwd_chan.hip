// Per-chunk gradients of the chunkwise gated delta rule with a per-channel gate
// (bf16 I/O, d_k = 128) on gfx950.  The sequential passes that give every chunk its
// entering state S and the gradient dS' of the state leaving it are in
// chunk_bwd.hip; this is the third pass.
//
// The pages print no gradients; these are the reverse-mode derivatives of the
// chunk form of "Moonshot AI's New Attention Architecture: Key Innovations
// Explained", §2 (the per-channel gate a_t over key channels) and §3
// Hardware-Friendly Algorithm, with the gate kept in the log domain (§5).  Per chunk
// (rows r = 0..63, channels c, g_rc the running sum of log a inside the chunk,
// g_read = g, or g_{r-1} when the erase reads the undecayed state):
//   forward   Kp = k e^{g_read},  Kd = k e^{g_63 - g}  (from the per-chunk transform)
//             X = V - Kp S,  Delta = T diag(beta) X,  P = lower_incl((q e^g)(k e^{-g})^T)
//   d_v side  dDelta = P^T dO + Kd dS',  dY = T^T dDelta,  dv = diag(beta) dY,
//             dA = -strict_lower(dY Delta^T),  dP = lower_incl(dO Delta^T)
//   d_k side  G_r  = sum_{j<r}  dA_rj k_j e^{g_read_r - g_j},  H_r  = sum_{j<=r} dP_rj k_j e^{g_r - g_j},
//             Gc_j = sum_{r>j}  beta_r dA_rj k_r e^{g_read_r - g_j},
//             Hc_j = sum_{r>=j} dP_rj q_r e^{g_r - g_j}     (all elementwise in the channel)
//             dq = H + e^g (dO S^T)
//             dk = beta G + Gc + Hc - beta e^{g_read} (dY S^T) + e^{g_63 - g} (Delta dS'^T)
//             dbeta_r = sum_v dY X + k_r . G_r
//   gate      dg_rc = q dq - k (Gc + Hc + e^{g_63 - g} Delta dS'^T)          (at row r)
//                   + k (beta G - beta e^{g_read} dY S^T)                  (at the row g_read reads)
//             dg_63 += sum_r k e^{g_63 - g} (Delta dS'^T) + e^{g_63} sum_v S dS'
//             d log a_s = sum_{r >= s} dg_r
//
// The four d_k-side sums carry a decay per channel, so they cannot take one
// factor per row as the scalar gate does.  They are split at the 16-row blocks:
// for output block R and input block J,
//   e^{g_r - g_j} = e^{g_r - g_eR} e^{g_eR - g_eJ} e^{g_eJ - g_j}    (e = last row of a block; G, H)
//   e^{g_r - g_j} = e^{g_sR - g_j} ... with s = first row             (Gc, Hc: e^{g_r - g_sR} on the operand)
// The operand factor (<= 1) goes into the operand tile, the block-to-block factor
// (<= 1, one per channel) rescales the MFMA accumulator between input blocks, and
// the output factor (at most 16 tokens of decay) is applied in fp32.  Each operand
// tile is held as two bf16 tiles, the value and its rounding residual (16 bits of
// mantissa together): in the suffix sums of d log a the row-side and column-side
// terms of every pair of tokens inside the suffix cancel, and with the operand
// rounded once to bf16 they cancel only to its 8 bits, which costs d log a about
// 2 % relative error on long sequences against 0.1 % with the residual.
//
// One workgroup of eight waves per chunk.  Phase 1 takes d_v in slices of QW
// columns (X, dDelta; Delta, dY; then the products accumulated over d_v); phase 2
// forms g, the decayed operand tiles and the d_k-side sums, and writes dq, dk,
// dbeta and d log a.  Every sum is in a fixed order (no atomics).
#include <type_traits>

#include "bwd_common.h"
#include "launchers.h"

namespace gdr {

namespace {

constexpr int CDK = 128;   // d_k of this kernel

// QW: d_v columns per phase-1 slice (32 or 64).
template <int QW>
struct ChanLayout {
  // phase 1
  static constexpr int LKP = ld_row(CDK);    // k e^{g_read}, k e^{g_63 - g}: rows
  static constexpr int LCT = ld_both(CH);    // T^T
  static constexpr int LCP = ld_tr(CH);      // P
  static constexpr int LVQ = ld_both(QW);    // v slice, then diag(beta) X
  static constexpr int LOQ = ld_both(QW);    // dO slice
  static constexpr int LSQ = ld_both(CDK);   // S^T, dS'^T slices [32][d_k]
  static constexpr int LRQ = ld_row(QW);     // Delta, dY
  static constexpr int LDQ = ld_tr(QW);      // dDelta
  static constexpr size_t O_KP = 0;
  static constexpr size_t O_KD = O_KP + size_t(CH) * LKP * 2;
  static constexpr size_t O_T = O_KD + size_t(CH) * LKP * 2;
  static constexpr size_t O_P = O_T + size_t(CH) * LCT * 2;
  static constexpr size_t O_V = O_P + size_t(CH) * LCP * 2;
  static constexpr size_t O_DO = O_V + size_t(CH) * LVQ * 2;
  static constexpr size_t O_S = O_DO + size_t(CH) * LOQ * 2;
  static constexpr size_t O_DS = O_S + size_t(QW) * LSQ * 2;
  static constexpr size_t O_DL = O_DS + size_t(QW) * LSQ * 2;
  static constexpr size_t O_DY = O_DL + size_t(CH) * LRQ * 2;
  static constexpr size_t O_DD = O_DY + size_t(CH) * LRQ * 2;
  static constexpr size_t END1 = O_DD + size_t(CH) * LDQ * 2;
  // phase 2 (over the phase-1 tiles)
  static constexpr int LG = CDK + 4;         // g, fp32
  static constexpr int LA = ld_both(CH);     // dA, dP
  static constexpr int LX = ld_tr(CDK);      // a decayed operand tile: value, residual
  static constexpr int LR = ld_row(CDK);     // raw k, q
  static constexpr size_t O_G = 0;
  static constexpr size_t O_A = O_G + size_t(CH) * LG * 4;
  static constexpr size_t O_PD = O_A + size_t(CH) * LA * 2;
  static constexpr size_t O_X0 = O_PD + size_t(CH) * LA * 2;   // k e^{g_eJ - g}, beta k e^{g_read - g_sR},
  static constexpr size_t O_X1 = O_X0 + size_t(CH) * LX * 2;   // q e^{g - g_sR} in turn (value, residual)
  static constexpr size_t O_RK = O_X1 + size_t(CH) * LX * 2;
  static constexpr size_t O_RQ = O_RK + size_t(CH) * LR * 2;
  static constexpr size_t END2 = O_RQ + size_t(CH) * LR * 2;
  // both phases: factor rows of the record (beta; e^{g_63} per channel), the
  // segment totals of the gate scan, and fixed slots of the reductions
  static constexpr size_t O_F = cmax(END1, END2);
  static constexpr size_t O_TOT = O_F + 6 * CH * 4;           // [4][d_k]
  static constexpr size_t O_RED = O_TOT + 4 * CDK * 4;
  // dbeta: [QW / 16][64] (sum_v dY X by 16-column tile), [8][64] (k . G by channel
  // tile); <dS', S> by wave [8][d_k]
  static constexpr size_t NRED = (QW / 16) * CH + 8 * CH + 8 * CDK;
  static constexpr size_t TOTAL = O_RED + NRED * 4;
};

template <int DV, int QW>
__global__ __launch_bounds__(512) void bwd_chunk_chan_kernel(BwdParams p) {
  typedef ChanLayout<QW> L;
  constexpr int DK = CDK;
  constexpr int NT = 512;
  constexpr int NQ = DV / QW;
  constexpr int VT = QW / 16;                  // 16-column tiles per slice
  constexpr int NTW = 4 * VT / 8;              // phase-1 tiles (row block, column tile) per wave
  constexpr int VPR = QW / 8;                  // 16-byte pieces per row of a v or dO slice
  constexpr int NVP = CH * VPR;                // ... per slice
  constexpr int NVO = 2 * NVP / NT;            // v and dO pieces per thread
  constexpr int NSP = QW * DK / 8 / NT;        // pieces of an S^T slice per thread
  static_assert(NTW >= 1 && NVO >= 1 && NSP >= 1 && NVP % 64 == 0, "slice width");
  constexpr uint32_t RB = rec_bytes(IO_BF16, GATE_CHANNEL, DK);
  constexpr uint32_t SBYTES = DV * DK * 2;
  static_assert(L::TOTAL <= 163840, "LDS budget");
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  T* sKp = reinterpret_cast<T*>(smem + L::O_KP);
  T* sKd = reinterpret_cast<T*>(smem + L::O_KD);
  T* sT = reinterpret_cast<T*>(smem + L::O_T);
  T* sP = reinterpret_cast<T*>(smem + L::O_P);
  T* sV = reinterpret_cast<T*>(smem + L::O_V);
  T* sdO = reinterpret_cast<T*>(smem + L::O_DO);
  T* sS = reinterpret_cast<T*>(smem + L::O_S);
  T* sdS = reinterpret_cast<T*>(smem + L::O_DS);
  T* sDl = reinterpret_cast<T*>(smem + L::O_DL);
  T* sdY = reinterpret_cast<T*>(smem + L::O_DY);
  T* sdD = reinterpret_cast<T*>(smem + L::O_DD);
  float* sG = reinterpret_cast<float*>(smem + L::O_G);
  T* sA = reinterpret_cast<T*>(smem + L::O_A);
  T* sPd = reinterpret_cast<T*>(smem + L::O_PD);
  T* sX0 = reinterpret_cast<T*>(smem + L::O_X0);
  T* sX1 = reinterpret_cast<T*>(smem + L::O_X1);
  T* sRk = reinterpret_cast<T*>(smem + L::O_RK);
  T* sRq = reinterpret_cast<T*>(smem + L::O_RQ);
  const float* sF = reinterpret_cast<const float*>(smem + L::O_F);   // beta [64], e^{g_63} [d_k]
  float* sTot = reinterpret_cast<float*>(smem + L::O_TOT);
  float* rbX = reinterpret_cast<float*>(smem + L::O_RED);
  float* rbK = rbX + VT * CH;
  float* rsd = rbK + 8 * CH;

  const ChunkParams& f = p.f;
  const int H = static_cast<int>(f.H);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const bool literal = f.literal != 0;

  int64_t bb, n, hh;
  if (!prep_task(f, blockIdx.x, bb, n, hh)) return;
  const BwdSeq sq = bwd_seq_of(f, bb, hh);
  const int64_t nch = sq.nch;
  const Slice sl = sq.sl;
  const rsrc_t rw = make_rsrc(static_cast<const char*>(f.ws) + sq.rec0 * RB, static_cast<uint32_t>(nch * RB));
  const rsrc_t rv = sl.rs(f.v, DV), rdo = sl.rs(p.dO, DV);
  const rsrc_t rst = make_rsrc(static_cast<const char*>(p.states) + sq.rec0 * SBYTES, static_cast<uint32_t>(nch * SBYTES));
  const rsrc_t rds = make_rsrc(static_cast<const char*>(p.dstates) + sq.rec0 * SBYTES, static_cast<uint32_t>(nch * SBYTES));
  const uint32_t sw = static_cast<uint32_t>(n * RB);
  const uint32_t sk = static_cast<uint32_t>(n * CH * H * DK * 2);   // chunk start in q, k, log a (bytes)
  const uint32_t sv = static_cast<uint32_t>(n * CH * H * DV * 2);   // ... in v, dO
  const uint32_t ss = static_cast<uint32_t>(n) * SBYTES;
  const uint32_t sb = static_cast<uint32_t>(n * CH * H * 2);        // ... in beta

  // ---- the record's decayed k tiles, T, P and factor rows ----------------------------
  {
    u32x4 hkp[2], hkd[2], ht, hp, hf;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t off = W::X_OFF + static_cast<uint32_t>((tid + i * NT) * 16);
      hkp[i] = buf_load16(rw, off, sw);
      hkd[i] = buf_load16(rw, off + 2 * CH * DK * 2, sw);
    }
    if (tid < 320) {
      ht = buf_load16(rw, W::T_OFF + static_cast<uint32_t>(tid * 16), sw);
      hp = buf_load16(rw, W::P_OFF + static_cast<uint32_t>(tid * 16), sw);
    }
    if (tid < 96) hf = buf_load16(rw, W::F_OFF + static_cast<uint32_t>(tid * 16), sw);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pc = tid + i * NT;   // row pc / 16, channels 8 (pc % 16) ..
      put16(sKp + (pc / 16) * L::LKP + (pc % 16) * 8, hkp[i]);
      put16(sKd + (pc / 16) * L::LKP + (pc % 16) * 8, hkd[i]);
    }
    if (tid < 320) {                 // block u: T_RJ transposed (into T^T) and P_RJ
      int R, J;
      tri_block(tid / 32, R, J);
      const int a = (tid % 32) / 2, b0 = (tid % 2) * 8;
      put16(sT + (16 * J + a) * L::LCT + 16 * R + b0, ht);
      put16(sP + (16 * R + a) * L::LCP + 16 * J + b0, hp);
    }
    if (tid < 96) *reinterpret_cast<u32x4*>(smem + L::O_F + tid * 16) = hf;
  }

  // ---- one slice of v, dO, S^T, dS'^T -----------------------------------------------
  // Piece pv = tid + i NT of the v and dO slices is dO's when pv >= NVP (the choice is
  // the same for the whole wave): row (pv % NVP) / VPR, columns 8 (pv % VPR) ..
  u32x4 hvo[NVO], hs[NSP], hds[NSP];
  float sdot[8];                      // this thread's part of sum_v S dS' for channels 8 (tid % 16) ..
#pragma unroll
  for (int e = 0; e < 8; ++e) sdot[e] = 0.f;
  auto load_slice = [&](int qi) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NVO; ++i) {
      const int t = (tid + i * NT) % NVP;
      const bool is_do = (64 * wave + i * NT) >= NVP;
      hvo[i] = buf_load16(is_do ? rdo : rv, static_cast<uint32_t>(((t / VPR) * H * DV + QW * qi + (t % VPR) * 8) * 2), sv);
    }
#pragma unroll
    for (int i = 0; i < NSP; ++i) {   // piece pc: column QW qi + pc / 16 of S, d_k values 8 (pc % 16) ..
      const int pc = tid + i * NT;
      const uint32_t off = chunk_state_off(8 * (pc % 16), QW * qi + pc / 16, DV);
      hs[i] = buf_load16(rst, off, ss);
      hds[i] = buf_load16(rds, off, ss);
    }
  };
  auto store_slice = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NVO; ++i) {
      const int t = (tid + i * NT) % NVP;
      const bool is_do = (64 * wave + i * NT) >= NVP;
      put16((is_do ? sdO : sV) + (t / VPR) * L::LVQ + (t % VPR) * 8, hvo[i]);
    }
#pragma unroll
    for (int i = 0; i < NSP; ++i) {
      const int pc = tid + i * NT;
      put16(sS + (pc / 16) * L::LSQ + (pc % 16) * 8, hs[i]);
      put16(sdS + (pc / 16) * L::LSQ + (pc % 16) * 8, hds[i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a = hs[i][j], b = hds[i][j];
        sdot[2 * j] += bf16_bits_to_f32(a & 0xffffu) * bf16_bits_to_f32(b & 0xffffu);
        sdot[2 * j + 1] += bf16_bits_to_f32(a >> 16) * bf16_bits_to_f32(b >> 16);
      }
    }
  };
  static_assert(L::LVQ == L::LOQ, "v and dO slices share a stride");

  // phase-2 inputs, fetched during the last slice: log a, k, q (row pc / 16, channels 8 (pc % 16) ..)
  u32x4 hla[2], hk[2], hq[2];
  auto load_phase2 = [&]() __attribute__((always_inline)) {
    const rsrc_t rla = sl.rs(f.log_a, DK), rk = sl.rs(f.k, DK), rq = sl.rs(f.q, DK);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pc = tid + i * NT;
      const uint32_t off = static_cast<uint32_t>(((pc / 16) * H * DK + (pc % 16) * 8) * 2);
      hla[i] = buf_load16(rla, off, sk);
      hk[i] = buf_load16(rk, off, sk);
      hq[i] = buf_load16(rq, off, sk);
    }
  };

  load_slice(0);
  store_slice();
  __syncthreads();

  // Phase-1 tiles of this wave: tiles t = wave + 8 i (row block t / VT, 16-column tile
  // t % VT of each slice) of X, dDelta, Delta and dY; the 64 x 64 blocks u = wave,
  // wave + 8 (< 10) of dA and dP; and, for the d_k-side products, channel tile `wave`
  // over all four row blocks.
  f32x4 dAa[2], dPa[2], dOS[4], dYS[4], DdS[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) dAa[i] = dPa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int R = 0; R < 4; ++R) dOS[R] = dYS[R] = DdS[R] = f32x4{0.f, 0.f, 0.f, 0.f};
  float bxp[NTW], beta1[NTW];          // sum_v dY X of the tile's row 16 R + lr; beta of that row
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    bxp[i] = 0.f;
    beta1[i] = sF[16 * ((wave + 8 * i) / VT) + lr];
  }
  const rsrc_t rdv = sl.rs(p.dv, DV);

  for (int qi = 0; qi < NQ; ++qi) {
    if (qi + 1 < NQ) load_slice(qi + 1);
    else load_phase2();
    // X and dDelta, row form (lane: row 16 R + lr, columns 16 vt + 4 lg ..)
    f32x4 x[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int R = (wave + 8 * i) / VT, vt = (wave + 8 * i) % VT;
      f32x4 xa = {0.f, 0.f, 0.f, 0.f}, dd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        xa = O::mma2(xa, rowf(sS, L::LSQ, 16 * vt, 32 * kb, lr, lg), rowf(sS, L::LSQ, 16 * vt, 32 * kb + 16, lr, lg),
                     rowf(sKp, L::LKP, 16 * R, 32 * kb, lr, lg), rowf(sKp, L::LKP, 16 * R, 32 * kb + 16, lr, lg));
        dd = O::mma2(dd, rowf(sdS, L::LSQ, 16 * vt, 32 * kb, lr, lg), rowf(sdS, L::LSQ, 16 * vt, 32 * kb + 16, lr, lg),
                     rowf(sKd, L::LKP, 16 * R, 32 * kb, lr, lg), rowf(sKd, L::LKP, 16 * R, 32 * kb + 16, lr, lg));
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)  // + P^T dO (rows of P from block R down)
        if (kb >= R) dd = O::mma1(dd, colf(sdO, L::LOQ, 16 * kb, 16 * vt, lr, lg), colf(sP, L::LCP, 16 * kb, 16 * R, lr, lg));
      x[i] = O::f32(rowf(sV, L::LVQ, 16 * R, 16 * vt, lr, lg)) - xa;   // X = V - Kp S
      st_row(sV, L::LVQ, 16 * R + lr, 16 * vt + 4 * lg, x[i] * beta1[i]);   // only this wave reads this tile of v
      st_row(sdD, L::LDQ, 16 * R + lr, 16 * vt + 4 * lg, dd);
    }
    __syncthreads();

    // Delta = T diag(beta) X and dY = T^T dDelta, row form
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int R = (wave + 8 * i) / VT, vt = (wave + 8 * i) % VT;
      f32x4 dl = {0.f, 0.f, 0.f, 0.f}, dy = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J <= R) dl = O::mma1(dl, colf(sV, L::LVQ, 16 * J, 16 * vt, lr, lg), colf(sT, L::LCT, 16 * J, 16 * R, lr, lg));
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        if (kb >= R) dy = O::mma1(dy, colf(sdD, L::LDQ, 16 * kb, 16 * vt, lr, lg), rowf(sT, L::LCT, 16 * R, 16 * kb, lr, lg));
      st_row(sDl, L::LRQ, 16 * R + lr, 16 * vt + 4 * lg, dl);
      st_row(sdY, L::LRQ, 16 * R + lr, 16 * vt + 4 * lg, dy);
      buf_store8(bits8(dy * beta1[i]), rdv, static_cast<uint32_t>(((16 * R + lr) * H * DV + QW * qi + 16 * vt + 4 * lg) * 2), sv);
      bxp[i] += lg_sum(dy[0] * x[i][0] + dy[1] * x[i][1] + dy[2] * x[i][2] + dy[3] * x[i][3]);
    }
    __syncthreads();

    // products over this slice's columns
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = wave + 8 * i;
      if (u < 10) {                    // row form: lane row 16R + lr of dY Delta^T and dO Delta^T
        int R, J;
        tri_block(u, R, J);
#pragma unroll
        for (int kk = 0; kk < QW / 32; ++kk) {
          const frag d0 = rowf(sDl, L::LRQ, 16 * J, 32 * kk, lr, lg), d1 = rowf(sDl, L::LRQ, 16 * J, 32 * kk + 16, lr, lg);
          dAa[i] = O::mma2(dAa[i], d0, d1, rowf(sdY, L::LRQ, 16 * R, 32 * kk, lr, lg),
                           rowf(sdY, L::LRQ, 16 * R, 32 * kk + 16, lr, lg));
          dPa[i] = O::mma2(dPa[i], d0, d1, rowf(sdO, L::LOQ, 16 * R, 32 * kk, lr, lg),
                           rowf(sdO, L::LOQ, 16 * R, 32 * kk + 16, lr, lg));
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < QW / 32; ++kk) {
      const frag s0 = colf(sS, L::LSQ, 32 * kk, 16 * wave, lr, lg), s1 = colf(sS, L::LSQ, 32 * kk + 16, 16 * wave, lr, lg);
      const frag e0 = colf(sdS, L::LSQ, 32 * kk, 16 * wave, lr, lg), e1 = colf(sdS, L::LSQ, 32 * kk + 16, 16 * wave, lr, lg);
#pragma unroll
      for (int R = 0; R < 4; ++R) {    // column form: rows 16R + 4 lg + s, channel 16 wave + lr
        dOS[R] = O::mma2(dOS[R], rowf(sdO, L::LOQ, 16 * R, 32 * kk, lr, lg), rowf(sdO, L::LOQ, 16 * R, 32 * kk + 16, lr, lg),
                         s0, s1);
        dYS[R] = O::mma2(dYS[R], rowf(sdY, L::LRQ, 16 * R, 32 * kk, lr, lg), rowf(sdY, L::LRQ, 16 * R, 32 * kk + 16, lr, lg),
                         s0, s1);
        DdS[R] = O::mma2(DdS[R], rowf(sDl, L::LRQ, 16 * R, 32 * kk, lr, lg), rowf(sDl, L::LRQ, 16 * R, 32 * kk + 16, lr, lg),
                         e0, e1);
      }
    }
    __syncthreads();
    if (qi + 1 < NQ) {
      store_slice();
      __syncthreads();
    }
  }

  // ---- phase 2: dA, dP, raw log a, k, q into LDS; reduction slots ----------------------
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = wave + 8 * i;
    if (u < 10) {
      int R, J;
      tri_block(u, R, J);
      const int r = 16 * R + lr;
      f32x4 a, pv;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int j = 16 * J + 4 * lg + s;
        a[s] = j < r ? -dAa[i][s] : 0.f;
        pv[s] = j <= r ? dPa[i][s] : 0.f;
      }
      st_row(sA, L::LA, r, 16 * J + 4 * lg, a);
      st_row(sPd, L::LA, r, 16 * J + 4 * lg, pv);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int pc = tid + i * NT, row = pc / 16, c0 = (pc % 16) * 8;
    float* gd = sG + row * L::LG + c0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      gd[2 * j] = bf16_bits_to_f32(hla[i][j] & 0xffffu);
      gd[2 * j + 1] = bf16_bits_to_f32(hla[i][j] >> 16);
    }
    put16(sRk + row * L::LR + c0, hk[i]);
    put16(sRq + row * L::LR + c0, hq[i]);
  }
#pragma unroll
  for (int i = 0; i < NTW; ++i)
    if (lg == 0) rbX[((wave + 8 * i) % VT) * CH + 16 * ((wave + 8 * i) / VT) + lr] = bxp[i];
#pragma unroll
  for (int e = 0; e < 8; ++e) {        // <dS', S> over this wave's rows of the slices
    const float v = lg_sum(sdot[e]);
    if (lg == 0) rsd[wave * DK + lr * 8 + e] = v;
  }
  __syncthreads();

  // ---- the gate: thread (channel cs, row block Rg) scans 16 rows and keeps them -------
  const int cs = tid & (DK - 1), Rg = tid >> 7;
  float gv[16], g0;                    // g of the 16 rows; g of the row before them (0 before the chunk)
  {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      acc += sG[(16 * Rg + j) * L::LG + cs];
      gv[j] = acc;
    }
    sTot[Rg * DK + cs] = acc;
    __syncthreads();
    g0 = 0.f;
    for (int R = 0; R < Rg; ++R) g0 += sTot[R * DK + cs];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      gv[j] += g0;
      sG[(16 * Rg + j) * L::LG + cs] = gv[j];
    }
  }
  // One decayed operand tile, as value and residual: k e^{g_eJ - g} (X = 0), beta k
  // e^{g_read - g_sR} (X = 1) or q e^{g - g_sR} (X = 2).
  auto form = [&](auto X) __attribute__((always_inline)) {
    float gp = g0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 16 * Rg + j;
      const float g = gv[j], grd = literal ? gp : g;
      gp = g;
      float x;
      if constexpr (decltype(X)::value == 0) x = static_cast<float>(sRk[r * L::LR + cs]) * __expf(gv[15] - g);
      else if constexpr (decltype(X)::value == 1) x = sF[r] * static_cast<float>(sRk[r * L::LR + cs]) * __expf(grd - gv[0]);
      else x = static_cast<float>(sRq[r * L::LR + cs]) * __expf(g - gv[0]);
      const T hi = O::from(x);
      sX0[r * L::LX + cs] = hi;
      sX1[r * L::LX + cs] = O::from(x - static_cast<float>(hi));
    }
  };
  form(std::integral_constant<int, 0>());
  __syncthreads();

  // ---- the d_k-side sums for channel tile `wave` (column form) --------------------------
  const int c = 16 * wave + lr;
  auto gat = [&](int r) __attribute__((always_inline)) { return sG[r * L::LG + c]; };
  f32x4 Ga[4], Ha[4], Gca[4], Hca[4];
#pragma unroll
  for (int R = 0; R < 4; ++R) {        // G, H: input blocks J = 0..R, block-end references
    f32x4 ag = {0.f, 0.f, 0.f, 0.f}, ah = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J <= R; ++J) {
      if (J > 0) {
        const float fj = __expf(gat(16 * J + 15) - gat(16 * J - 1));
        ag = ag * fj;
        ah = ah * fj;
      }
      const frag x0 = colf(sX0, L::LX, 16 * J, 16 * wave, lr, lg), x1 = colf(sX1, L::LX, 16 * J, 16 * wave, lr, lg);
      const frag a = rowf(sA, L::LA, 16 * R, 16 * J, lr, lg), pd = rowf(sPd, L::LA, 16 * R, 16 * J, lr, lg);
      ag = O::mma1(O::mma1(ag, a, x0), a, x1);
      ah = O::mma1(O::mma1(ah, pd, x0), pd, x1);
    }
    Ga[R] = ag;
    Ha[R] = ah;
  }
  // Gc (X = 1, with dA) and Hc (X = 2, with dP): input blocks R = 3..J, block-start references
  auto colside = [&](const T* sM, f32x4* out) __attribute__((always_inline)) {
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4 ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int R = 3; R >= J; --R) {
        if (R < 3) ag = ag * __expf(gat(16 * R + 16) - gat(16 * R));
        const frag m = colf(sM, L::LA, 16 * R, 16 * J, lr, lg);
        ag = O::mma1(O::mma1(ag, m, colf(sX0, L::LX, 16 * R, 16 * wave, lr, lg)), m,
                     colf(sX1, L::LX, 16 * R, 16 * wave, lr, lg));
      }
      out[J] = ag;
    }
  };
  __syncthreads();
  form(std::integral_constant<int, 1>());
  __syncthreads();
  colside(sA, Gca);
  __syncthreads();
  form(std::integral_constant<int, 2>());
  __syncthreads();
  colside(sPd, Hca);

  // ---- dq, dk, the gate terms per element; dbeta's k . G -------------------------------
  const rsrc_t rdq = sl.rs(p.dq, DK), rdk = sl.rs(p.dk, DK), rdl = sl.rs(p.dlog_a, DK);
  const float g63 = gat(63);
  float own[4][4], rdt[4][4];          // dg at row r, and the terms of the row g_read reads
  float c63 = 0.f;                     // sum_r k e^{g_63 - g} (Delta dS'^T)
#pragma unroll
  for (int R = 0; R < 4; ++R) {
    const float gsR = gat(16 * R), geR = gat(16 * R + 15);
    float kg[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = 16 * R + 4 * lg + s;
      const float g = gat(r);
      const float grd = literal ? (r > 0 ? gat(r - 1) : 0.f) : g;
      const float be = sF[r];
      const float kk = static_cast<float>(sRk[r * L::LR + c]), qq = static_cast<float>(sRq[r * L::LR + c]);
      const float Gv = __expf(grd - geR) * Ga[R][s];
      const float Hv = __expf(g - geR) * Ha[R][s];
      const float eo = __expf(gsR - g);
      const float Cv = eo * (Gca[R][s] + Hca[R][s]);
      const float dqv = Hv + __expf(g) * dOS[R][s];
      const float dkx = -be * __expf(grd) * dYS[R][s];
      const float kdt = __expf(g63 - g) * DdS[R][s];
      const float dkv = be * Gv + Cv + dkx + kdt;
      own[R][s] = qq * dqv - kk * (Cv + kdt);
      rdt[R][s] = kk * (be * Gv + dkx);
      c63 += kk * kdt;
      kg[s] = kk * Gv;
      const uint32_t off = static_cast<uint32_t>((r * H * DK + c) * 2);
      buf_store2(f32_to_bf16_bits(dqv), rdq, off, sk);
      buf_store2(f32_to_bf16_bits(dkv), rdk, off, sk);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {      // sum over the wave's 16 channels, one slot per row
      const float v = row16_sum(kg[s]);
      if (lr == 0) rbK[wave * CH + 16 * R + 4 * lg + s] = v;
    }
  }

  // ---- d log a: suffix sums over the chunk's rows, per channel ---------------------------
  c63 = lg_sum(c63);
  float sds = 0.f;                     // <dS', S> of channel c
  for (int w = 0; w < 8; ++w) sds += rsd[w * DK + c];
  const float tail63 = c63 + sF[CH + c] * sds;   // terms of g_63: every row s <= 63 takes them
  float t[4][4], bt[4];
#pragma unroll
  for (int R = 0; R < 4; ++R) {        // within the lane: rows 16R + 4 lg + s, s = 3..0
    float a = 0.f;
#pragma unroll
    for (int s = 3; s >= 0; --s) {
      a += own[R][s] + rdt[R][s];
      t[R][s] = a;
    }
    bt[R] = a;
  }
  float tail = tail63;                 // sum over the row blocks below
#pragma unroll
  for (int R = 3; R >= 0; --R) {
    const float b0 = __shfl(bt[R], lr), b1 = __shfl(bt[R], lr + 16), b2 = __shfl(bt[R], lr + 32),
                b3 = __shfl(bt[R], lr + 48);
    const float below = (lg < 1 ? b1 : 0.f) + (lg < 2 ? b2 : 0.f) + (lg < 3 ? b3 : 0.f);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = 16 * R + 4 * lg + s;
      const float d = t[R][s] + below + tail - (literal ? rdt[R][s] : 0.f);
      buf_store2(f32_to_bf16_bits(d), rdl, static_cast<uint32_t>((r * H * DK + c) * 2), sk);
    }
    tail += ((b0 + b1) + b2) + b3;
  }
  __syncthreads();

  // ---- dbeta -----------------------------------------------------------------------------
  if (wave == 0) {
    float d = 0.f;
    for (int v = 0; v < VT; ++v) d += rbX[v * CH + lane];
    for (int w = 0; w < 8; ++w) d += rbK[w * CH + lane];
    const rsrc_t rdb = sl.rs(p.dbeta, 1);
    buf_store2(f32_to_bf16_bits(d), rdb, static_cast<uint32_t>(lane * H * 2), sb);
  }
}

}  // namespace

hipError_t launch_chunk_bwd_chan(const BwdParams& p, hipStream_t stream) {
  const ChunkParams& f = p.f;
  if (f.d_k != CDK) return hipErrorInvalidValue;
  const int64_t nch = (f.T + CH - 1) / CH;
  const unsigned grid = static_cast<unsigned>(f.cu ? f.H * f.nslots : f.B * f.H * nch);
  // 32-column slices: 64-column ones halve phase 1's barriers but spill at d_v = 128
  // and measured slower (5.92 against 5.74 ms per call on B2 H32 T32768).
  if (f.d_v == 128)
    hipLaunchKernelGGL((bwd_chunk_chan_kernel<128, 32>), dim3(grid), dim3(512), 0, stream, p);
  else if (f.d_v == 64)
    hipLaunchKernelGGL((bwd_chunk_chan_kernel<64, 32>), dim3(grid), dim3(512), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gdr
