// Inter-chunk state scan: decayed chunk-boundary states of H and G.
//
// MesaNet page, technical summary, "Mesa layer" section, parallelisation
// paragraph: the layer keeps the states G_t, H_t and solves the per-token
// systems chunk by chunk.  Within a chunk c of tokens s..e the recurrence
// H_t = gamma_t H_{t-1} + beta_t k_t k_t^T folds into
//
//     H_e = Gamma_c H_{s-1} + K^T diag(beta .* tail) K,
//     Gamma_c = prod_{i=s..e} gamma_i,  tail_j = prod_{i=j+1..e} gamma_i,
//
// and the same for G with V^T in place of the first K^T.  This kernel walks
// the chunks of one (b, h) in order, keeps the running state in fp32
// registers, and writes the state *before* each chunk (the boundary state
// the CG kernel starts from) into the workspace.
//
// Work split: a workgroup owns either a whole state (H or G) of one (b, h)
// -- FULL, 8 waves -- or one 16-row stripe of it (4 waves), so there are 2 or 2*D/16
// workgroups per (b, h); the launch picks the split that fills the GPU and
// maps the workgroups of one (b, h) onto one XCD (they share the chunk's keys
// in that XCD's L2).  The keys, values and gates of the chunk after next are
// loaded into registers while the current chunk is processed, and the staged
// operands alternate between two LDS buffers, so a chunk costs one barrier.  The chunk delta
// K^T diag(w) X is an MFMA contraction over the chunk's tokens: bf16 MFMA for
// bf16 inputs with the scaled operand split into bf16 hi + lo parts (so the
// carried fp32 state does not pick up a bf16 rounding of beta*tail*x), fp32
// MFMA for fp32 inputs.
//
// PREP (fused preprocessing, bf16, chunk 64): the keys arrive raw and are
// convolved and L2-normalised as they are staged (mesa_prep_rows.h: a row's
// D/8 lanes side by side, the same arithmetic as the preprocessing kernel).
// Each group of D/8 lanes forms RPG consecutive rows of the chunk from the
// RPG + 3 raw rows that end at them, prefetched like the other operands, and
// stores them row-major in LDS (16 bytes per lane, whole rows per group: a
// direct transposed store from this layout would put a group's lanes 8 rows
// of the transposed array apart, all in one bank).  After a barrier the
// plain path's pieces are read back from there and staged exactly as the
// plain path stages loaded keys, so the processed keys never reach HBM.
//
// Snapshot layouts (consumed only by the CG kernels):
//   fp32 path: row-major [D][D] fp32, H[r][c] and G[v][k].
//   bf16 path: MFMA A-operand fragments.  Fragment f = nt*(D/32) + m holds,
//     for lane l (tl = l%16, g = l/16), 8 bf16: row 16*nt + tl, columns
//     32m + 4g + {0..3} then 32m + 16 + 4g + {0..3}.  Stored [f][lane][8].
#include "mesa_common.h"
#include "mesa_kernels.h"
#include "mesa_prep_rows.h"

namespace mesa {

namespace {


template <bool BF16, int D, int C, bool FULL, bool PREP = false>
struct ScanShape {
  static constexpr int ND = D / 16;
  static constexpr int CP = (C < 32) ? 32 : C;       // token dim padded to one bf16 k-block
  static constexpr int U = FULL ? 2 : 2 * ND;          // workgroups per (b, h)
  static constexpr int MROWS = FULL ? D : 16;          // state rows (A-operand rows) owned
  static constexpr bool PAIR = FULL && BF16;           // a unit = both m-tiles of a fragment
  static constexpr int TPU = PAIR ? 2 : 1;             // tiles per unit
  static constexpr int NU = FULL ? (PAIR ? (ND / 2) * ND : ND * ND) : ND;
  // a whole state per workgroup takes 8 waves, a stripe 4 (state and
  // prefetch registers per thread stay well under the VGPR file)
  static constexpr int THREADS = FULL ? 512 : 256;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int UPW = (NU + WAVES - 1) / WAVES; // units per wave
  // every wave owns exactly UPW units (no guard, so no divergent branch
  // in the chunk loop: a branch join there costs the loads' wait counts)
  static constexpr bool EVEN = NU % WAVES == 0;
  // register prefetch: pieces of the chunk each thread loads
  static constexpr int NPX = BF16 ? (CP / 2) * (D / 8) : C * (D / 4);   // X pieces
  static constexpr int PPX = (NPX + THREADS - 1) / THREADS;
  static constexpr int NPK = BF16 ? (CP / 2) * (MROWS / 8) : C * (MROWS / 4);  // K pieces (A operand)
  static constexpr int PPK = (NPK + THREADS - 1) / THREADS;
  static constexpr int AS = CP + 8;                    // bf16 row stride of transposed LDS arrays
  static constexpr size_t LDS_A = BF16 ? (size_t)MROWS * AS * 2 : (size_t)CP * MROWS * 4;
  static constexpr size_t LDS_B = BF16 ? (size_t)2 * D * AS * 2 : (size_t)CP * D * 4;
  // PREP: lanes per key row; PG groups of them form the chunk's rows, RPG
  // consecutive rows each, from NRR raw rows per lane
  static constexpr int LPR = D / 8;
  static constexpr int PG = (THREADS / LPR < C) ? THREADS / LPR : C;
  static constexpr int RPG = C / PG;
  static constexpr int NRR = PREP ? RPG + kPrepMaxW - 1 : 1;
  static constexpr int PSS = D + 8;  // bf16 row stride of the processed keys (16-byte rows, 2-way reads)
  // PREP with a whole state (PF): each X piece (rows 2jp, 2jp+1, channels
  // 8c8..8c8+7) is convolved by the lane that stages it, from its 5 raw rows
  // 2jp-3 .. 2jp+1; the row norms come from per-channel-group partial sums in
  // LDS, SSB floats per row pair (2 rows x D/8 groups + 16 bytes of padding,
  // so that 8 lanes' 16-byte reads of consecutive pairs hit distinct banks)
  static constexpr bool PF = PREP && FULL;
  static constexpr int NKR = PF ? 5 * PPX : NRR;
  static constexpr int SSB = 2 * (D / 8) + 4;
};

// Two floats rounded to bf16 (nearest even) and packed low-first into one
// dword by one paired conversion (single conversions need a merge each).
__device__ __forceinline__ uint32_t cvt_pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <bool BF16>
struct Piece;
template <>
struct Piece<true> { u16x8 a, b; };   // two token rows (j0, j1), 8 columns each
template <>
struct Piece<false> { f32x4 a; };     // one token row, 4 columns

// TOTALS: the first pass of a segmented walk -- each segment from a zero
// state, no snapshots, the segment's total state and decay at the end.
template <bool BF16, int D, int C, bool FULL, bool TOTALS, bool PREP = false>
__global__ __launch_bounds__((ScanShape<BF16, D, C, FULL>::THREADS)) void scan_kernel(ScanParams p) {
  using S = ScanShape<BF16, D, C, FULL, PREP>;
  static_assert(!PREP || (BF16 && C == 64 && S::PG * S::RPG == C), "fused preprocessing: bf16, chunk 64");
  constexpr int ND = S::ND, CP = S::CP, U = S::U, MROWS = S::MROWS, TPU = S::TPU, UPW = S::UPW;
  constexpr int AS = S::AS;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, tl = lane & 15, g = lane >> 4;

  // XCD-aware decode: the workgroups of one (b, h) share blockIdx % 8.
  // Within an XCD: (b, h) group, then segment, then unit.
  const int NSP = TOTALS ? p.NS - 1 : p.NS;  // segments walked by this launch
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  const int u0 = local % U;
  const int seg = (local / U) % NSP;
  const int bh = (local / U / NSP) * 8 + xcd;
  if (bh >= p.BH) return;
  const int which = FULL ? u0 : u0 / ND;   // 0: H, 1: G
  const int mpart = FULL ? 0 : u0 % ND;    // stripe (non-FULL)
  const int T = p.T, NC = p.NC;
  const int cb = seg * p.SEG, ce = min(cb + p.SEG, NC);  // this segment's chunks
  const void* X = which ? p.v : p.k;      // the second factor of the chunk delta
  const size_t rowbase = (size_t)bh * T;

  // operand staging, double-buffered by chunk parity: one barrier per chunk
  __shared__ __attribute__((aligned(16))) char lds_a2[2][S::LDS_A];
  __shared__ __attribute__((aligned(16))) char lds_b2[2][S::LDS_B];

  // ---- ownership: unit list of this wave ----------------------------------------
  auto unit_mt = [&](int u, int h) -> int {
    if constexpr (FULL) return S::PAIR ? 2 * (u / ND) + h : u / ND;
    else return mpart;
  };
  auto unit_nt = [&](int u) -> int { return FULL ? u % ND : u; };

  // Running state: lane holds O[16 mt + 4 g + i][16 nt + tl], O = H (H) or G^T (G).
  f32x4 st[UPW][TPU];
  // start state: h0/g0 for the first segment, the carry-in state for a later
  // one (second pass), zero for a segment total
  const float* init = TOTALS ? nullptr : (seg == 0 ? (which ? p.g0 : p.h0) : p.seg_state);
  const size_t init_off = (TOTALS || seg == 0)
                              ? (size_t)bh * D * D
                              : (((size_t)bh * 2 + which) * (p.NS - 1) + (seg - 1)) * D * D;
  // (the source and layout are chosen per workgroup, so the state's loads are
  // issued as one batch)
#pragma unroll
  for (int ui = 0; ui < UPW; ++ui)
#pragma unroll
    for (int h = 0; h < TPU; ++h) st[ui][h] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (init) {
    const float* base = init + init_off;
    if (which == 0) {
#pragma unroll
      for (int ui = 0; ui < UPW; ++ui)
#pragma unroll
        for (int h = 0; h < TPU; ++h) {
          const int u = wave + S::WAVES * ui;
          const int mt = unit_mt(u, h), nt = unit_nt(u);
          if (S::EVEN || u < S::NU) {
#pragma unroll
            for (int i = 0; i < 4; ++i) st[ui][h][i] = base[(size_t)(16 * mt + 4 * g + i) * D + 16 * nt + tl];
          }
        }
    } else {
#pragma unroll
      for (int ui = 0; ui < UPW; ++ui)
#pragma unroll
        for (int h = 0; h < TPU; ++h) {
          const int u = wave + S::WAVES * ui;
          const int mt = unit_mt(u, h), nt = unit_nt(u);
          if (S::EVEN || u < S::NU)
            st[ui][h] = *reinterpret_cast<const f32x4*>(base + (size_t)(16 * nt + tl) * D + 16 * mt + 4 * g);
        }
    }
  }

  // ---- register prefetch of one chunk -------------------------------------------
  struct Raw {
    Piece<BF16> x[S::PPX];
    Piece<BF16> k[S::PPK];
    u16x8 kr[S::NKR];   // PREP: raw key rows (whole state: 2jp-3 .. 2jp+1 per piece;
                        // stripes: j0-3 .. j0+RPG-1 of this lane's group)
    float lg, bt;
  };
  // PREP: this lane's group of D/8 lanes (groups past PG -- whole waves --
  // form no rows), its first row and its channels; the head's taps sit in LDS
  // as [D][kPrepMaxW] (zero past W), read back at staging
  const int pgrp = tid / S::LPR, pc0 = 8 * (tid % S::LPR), pj0 = pgrp * S::RPG;
  const bool prow = PREP && (S::PG * S::LPR == S::THREADS || pgrp < S::PG);
  __shared__ __attribute__((aligned(16))) float ptap_s[PREP ? D * kPrepMaxW : 1];
  __shared__ __attribute__((aligned(16))) __bf16 prow_s[(PREP && !FULL) ? C * S::PSS : 1];  // processed keys [C][PSS]
  __shared__ __attribute__((aligned(16))) float ssp_s[S::PF ? 2 * (CP / 2) * S::SSB : 1];  // partials by chunk parity
  float yk[S::PF ? S::PPX : 1][2][8];  // PF: the next chunk's convolved keys, rows 2jp and 2jp+1 of each piece
  if constexpr (PREP) {
    for (int i = tid; i < D * kPrepMaxW; i += S::THREADS) {
      const int ch = i / kPrepMaxW, tap = i % kPrepMaxW;
      ptap_s[i] = tap < p.W ? p.wk[((size_t)(bh % p.H) * D + ch) * p.W + tap] : 0.f;
    }
    __syncthreads();
  }
  // Every load is unconditional (indices clamped into the chunk and the piece
  // list) so a fetch never waits on memory: the loads land while the previous
  // chunk is processed.  Rows past the chunk end repeat its last row; their
  // weight w_j is 0 (beta is taken as 0 there), so they add nothing.  The
  // raw gamma is kept; its log is taken when the chunk is processed.
  auto fetch = [&](int c, Raw& r) {
    const int s = c * C, Lc = min(C, T - s);
    const int jl = min(lane, Lc - 1);
    r.lg = p.gamma[rowbase + s + jl];
    r.bt = p.beta[rowbase + s + jl];
    auto row = [&](int j) { return rowbase + s + min(j, Lc - 1); };
    if constexpr (PREP) {
      // raw key rows of this lane's group (the previous rows for the window)
      // and the X pieces as the plain path loads them (for G the values; for
      // H, whose X is the processed keys formed at staging, raw keys that go
      // unused -- loaded all the same, so that no branch sits among the loads)
      const uint16_t* Xg = static_cast<const uint16_t*>(X);
      const uint16_t* Kg = static_cast<const uint16_t*>(p.k);
      const uint16_t* Kh = static_cast<const uint16_t*>(p.k_hist);
#pragma unroll
      for (int q = 0; q < S::PPX; ++q) {
        const int pc = min(tid + q * S::THREADS, S::NPX - 1);
        const int jp = pc % (CP / 2), c8 = pc / (CP / 2);
        r.x[q].a = *reinterpret_cast<const u16x8*>(Xg + row(2 * jp) * D + 8 * c8);
        r.x[q].b = *reinterpret_cast<const u16x8*>(Xg + row(2 * jp + 1) * D + 8 * c8);
      }
      if constexpr (S::PF) {
#pragma unroll
        for (int q = 0; q < S::PPX; ++q) {
          const int pc = min(tid + q * S::THREADS, S::NPX - 1);
          const int jp = pc % (CP / 2), c8 = pc / (CP / 2);
#pragma unroll
          for (int m = 0; m < 5; ++m)
            r.kr[5 * q + m] = prep_load8_w(Kg, Kh, bh, T, D, p.W, min(s + 2 * jp - 3 + m, s + Lc - 1), 8 * c8);
        }
      } else if (prow) {
#pragma unroll
        for (int m = 0; m < S::NRR; ++m)
          r.kr[m] = prep_load8_w(Kg, Kh, bh, T, D, p.W, min(s + pj0 - (kPrepMaxW - 1) + m, s + Lc - 1), pc0);
      }
    } else if constexpr (BF16) {
      const uint16_t* Xg = static_cast<const uint16_t*>(X);
      const uint16_t* Kg = static_cast<const uint16_t*>(p.k);
#pragma unroll
      for (int q = 0; q < S::PPX; ++q) {
        const int pc = min(tid + q * S::THREADS, S::NPX - 1);
        const int jp = pc % (CP / 2), c8 = pc / (CP / 2);
        r.x[q].a = *reinterpret_cast<const u16x8*>(Xg + row(2 * jp) * D + 8 * c8);
        r.x[q].b = *reinterpret_cast<const u16x8*>(Xg + row(2 * jp + 1) * D + 8 * c8);
      }
#pragma unroll
      for (int q = 0; q < S::PPK; ++q) {
        const int pc = min(tid + q * S::THREADS, S::NPK - 1);
        const int jp = pc % (CP / 2), c8 = pc / (CP / 2);
        const int col = (FULL ? 0 : 16 * mpart) + 8 * c8;
        r.k[q].a = *reinterpret_cast<const u16x8*>(Kg + row(2 * jp) * D + col);
        r.k[q].b = *reinterpret_cast<const u16x8*>(Kg + row(2 * jp + 1) * D + col);
      }
    } else {
      const float* Xg = static_cast<const float*>(X);
      const float* Kg = static_cast<const float*>(p.k);
#pragma unroll
      for (int q = 0; q < S::PPX; ++q) {
        const int pc = min(tid + q * S::THREADS, S::NPX - 1);
        const int j = pc / (D / 4), c4 = pc % (D / 4);
        r.x[q].a = *reinterpret_cast<const f32x4*>(Xg + row(j) * D + 4 * c4);
      }
#pragma unroll
      for (int q = 0; q < S::PPK; ++q) {
        const int pc = min(tid + q * S::THREADS, S::NPK - 1);
        const int j = pc / (MROWS / 4), c4 = pc % (MROWS / 4);
        const int col = (FULL ? 0 : 16 * mpart) + 4 * c4;
        r.k[q].a = *reinterpret_cast<const f32x4*>(Kg + row(j) * D + col);
      }
    }
  };

  // A ring of DEPTH chunk buffers: chunk c + DEPTH - 1 is fetched while chunk
  // c is processed, so each fetch has DEPTH - 1 chunk steps to land (three
  // buffers for bf16 inputs; two for fp32, whose buffers are twice as large).
  // The loop is unrolled by DEPTH so the buffers never move between
  // registers (a move would wait for the fetch), and every fetch is
  // unconditional (the chunk index is clamped; a fetch past the end is
  // simply not used).
  constexpr int DEPTH = BF16 ? 3 : 2;
  Raw b0, b1, b2;
  if (ce > cb) {
    fetch(cb, b0);
    if constexpr (DEPTH == 3) fetch(min(cb + 1, ce - 1), b1);
  }
  // ---- the bf16 snapshot of the current state as the state before chunk c ------
  auto store_snapshot = [&](const int c) {
    if constexpr (!TOTALS) {
      const size_t snap = ((size_t)bh * NC + c) * D * D;
#pragma unroll
      for (int ui = 0; ui < UPW; ++ui) {
        const int u = wave + S::WAVES * ui;
        if (!S::EVEN && u >= S::NU) continue;
        const int nt = unit_nt(u);
        if constexpr (BF16) {
          __bf16* dst = static_cast<__bf16*>(which ? p.gb : p.hb) + snap;
          if constexpr (S::PAIR) {
            const int frag = nt * (ND / 2) + u / ND;
            *reinterpret_cast<bf16x8*>(dst + ((size_t)frag * 64 + lane) * 8) = pack8(st[ui][0], st[ui][1]);
          } else {
            const int mt = unit_mt(u, 0);
            const int frag = nt * (ND / 2) + (mt >> 1);
            bf16x4 h4;
#pragma unroll
            for (int i = 0; i < 4; ++i) h4[i] = (__bf16)st[ui][0][i];
            *reinterpret_cast<bf16x4*>(dst + ((size_t)frag * 64 + lane) * 8 + 4 * (mt & 1)) = h4;
          }
        } else {
          float* dst = static_cast<float*>(which ? p.gb : p.hb) + snap;
#pragma unroll
          for (int h = 0; h < TPU; ++h) {
            const int mt = unit_mt(u, h);
            if (which == 0) {
#pragma unroll
              for (int i = 0; i < 4; ++i) dst[(size_t)(16 * mt + 4 * g + i) * D + 16 * nt + tl] = st[ui][h][i];
            } else {
              *reinterpret_cast<f32x4*>(dst + (size_t)(16 * nt + tl) * D + 16 * mt + 4 * g) = st[ui][h];
            }
          }
        }
      }
    }
  };
  if constexpr (FULL)
    if (ce > cb) store_snapshot(cb);
  // PF: convolve chunk c1's keys from its raw rows (raw), keep them in yk and
  // publish each row's channel-group partial sums of squares (ssp_s by chunk
  // parity) for the next step, which scales and stages them after the barrier
  auto conv_next = [&](const int c1, const Raw& raw) {
    if constexpr (S::PF) {
#pragma unroll
      for (int q = 0; q < S::PPX; ++q) {
        const int pc = tid + q * S::THREADS;
        if (S::NPX % S::THREADS != 0 && pc >= S::NPX) continue;  // whole waves
        const int jp = pc % (CP / 2), c8 = pc / (CP / 2);
        float w[8][kPrepMaxW];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(ptap_s + (8 * c8 + e) * kPrepMaxW);
#pragma unroll
          for (int i = 0; i < kPrepMaxW; ++i) w[e][i] = t4[i];
        }
        float* ssp = ssp_s + ((c1 & 1) * (CP / 2) + jp) * S::SSB;
        prep_with_window(p.W, [&](auto wc) {
          constexpr int WW = decltype(wc)::value;
#pragma unroll
          for (int rr = 0; rr < 2; ++rr) {
            const int j = 2 * jp + rr;
            float x8[kPrepMaxW][8];
#pragma unroll
            for (int m = kPrepMaxW - WW; m < kPrepMaxW; ++m)
              prep_unpack8(prep_zero_row(raw.kr[5 * q + rr + m], p.k_hist, p.W, c1 * C + j - (kPrepMaxW - 1) + m),
                           x8[m]);
            ssp[rr * (D / 8) + c8] = prep_conv8_pad<WW>(w, x8, yk[q][rr]);
          }
        });
      }
    }
  };
  if constexpr (S::PF) {
    if (ce > cb) conv_next(cb, b0);
    __syncthreads();
  }
  float seg_log = 0.f;  // sum of log gamma over the segment (wave-uniform)
  auto step = [&](const int c, const Raw& cur, const Raw& nxt, Raw& pre) {
    fetch(min(c + DEPTH - 1, ce - 1), pre);

    // the state before chunk c (stripes: stored here; whole or segment
    // states: stored right after chunk c-1's update, see below)
    if constexpr (!FULL) store_snapshot(c);

    // ---- gates (every wave, in registers): w_j = beta_j prod_{i>j} gamma_i ------
    const int Lcur = min(C, T - c * C);
    float suf = lane < Lcur ? logf(cur.lg) : 0.f;  // inclusive suffix sum of log gamma
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_down(suf, o, 64);
      if (lane + o < 64) suf += t;
    }
    // sum over i > j; the shuffle runs with every lane active, then lane 63 drops it
    const float next = __shfl_down(suf, 1, 64);
    const float after = (lane < 63) ? next : 0.f;
    const float wj = lane < Lcur ? cur.bt * expf(after) : 0.f;          // 0 past the chunk end
    const float sum_log = __shfl(suf, 0, 64);
    const float gamma_c = expf(sum_log);
    seg_log += sum_log;

    // ---- stage operands into the buffer of chunk parity c & 1: every wave
    // finished chunk c-2's products, which read it, before chunk c-1's barrier
    char* lds_a = lds_a2[c & 1];
    char* lds_b = lds_b2[c & 1];
    // bf16 staging from the X and K pieces: (w .* X)^T split into bf16 hi and
    // lo parts, and K^T of the owned stripe
    auto stage_bf16 = [&](const auto* xp, const auto* kp) {
      __bf16* KT = reinterpret_cast<__bf16*>(lds_a);  // [MROWS][AS]: K^T rows of the owned stripe
      __bf16* XH = reinterpret_cast<__bf16*>(lds_b);  // [D][AS]: (w .* X)^T, hi part
      __bf16* XL = XH + D * AS;                       // lo part
#pragma unroll
      for (int q = 0; q < S::PPX; ++q) {
        const int pc = tid + q * S::THREADS;
        const int jp = pc % (CP / 2), c8 = pc / (CP / 2);
        // shuffles before any lane leaves: every lane of the wave participates
        const float w0 = __shfl(wj, (2 * jp) & 63, 64), w1 = __shfl(wj, (2 * jp + 1) & 63, 64);
        if (S::NPX % S::THREADS != 0 && pc >= S::NPX) continue;
        const float ww0 = (2 * jp < C) ? w0 : 0.f, ww1 = (2 * jp + 1 < C) ? w1 : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x0 = ww0 * bf16_to_f32(xp[q].a[e]), x1 = ww1 * bf16_to_f32(xp[q].b[e]);
          // hi parts, then lo = x - hi rounded: two paired conversions
          const uint32_t hp = cvt_pack2(x0, x1);
          const uint32_t lp = cvt_pack2(x0 - __uint_as_float(hp << 16), x1 - __uint_as_float(hp & 0xffff0000u));
          const int n = 8 * c8 + e;
          *reinterpret_cast<uint32_t*>(XH + n * AS + 2 * jp) = hp;
          *reinterpret_cast<uint32_t*>(XL + n * AS + 2 * jp) = lp;
        }
      }
#pragma unroll
      for (int q = 0; q < S::PPK; ++q) {
        const int pc = tid + q * S::THREADS;
        if (S::NPK % S::THREADS != 0 && pc >= S::NPK) continue;
        const int jp = pc % (CP / 2), c8 = pc / (CP / 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = 8 * c8 + e;
          *reinterpret_cast<uint32_t*>(KT + m * AS + 2 * jp) =
              (uint32_t)kp[q].a[e] | ((uint32_t)kp[q].b[e] << 16);
        }
      }
    };
    if constexpr (S::PF) {
      // chunk c's keys: the row norms from the partial sums (summed in the
      // order of group_sum over a row's D/8 lanes), scaled and rounded as the
      // preprocessing kernel does, then staged as loaded keys are; then the
      // next chunk's convolution, published by this step's barrier
      Piece<BF16> xk[S::PPX], kk[S::PPX];
#pragma unroll
      for (int q = 0; q < S::PPX; ++q) {
        const int pc = min(tid + q * S::THREADS, S::NPX - 1);
        const int jp = pc % (CP / 2);
        const float* ssp = ssp_s + ((c & 1) * (CP / 2) + jp) * S::SSB;
        float part[2 * (D / 8)];
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(ssp + 4 * i);
#pragma unroll
          for (int u = 0; u < 4; ++u) part[4 * i + u] = t4[u];
        }
        const float sc0 = prep_scale(prep_tree_sum<D / 8>(part), p.inv_eps);
        const float sc1 = prep_scale(prep_tree_sum<D / 8>(part + D / 8), p.inv_eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kk[q].a[e] = __builtin_bit_cast(uint16_t, (__bf16)(yk[q][0][e] * sc0));
          kk[q].b[e] = __builtin_bit_cast(uint16_t, (__bf16)(yk[q][1][e] * sc1));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xk[q].a[e] = which ? cur.x[q].a[e] : kk[q].a[e];
          xk[q].b[e] = which ? cur.x[q].b[e] : kk[q].b[e];
        }
      }
      stage_bf16(xk, kk);
      conv_next(c + 1, nxt);
    } else if constexpr (PREP) {
      // the processed keys of the chunk, row-major in prow_s (each lane
      // group's 16-byte stores fill whole rows), then the same pieces the
      // plain path loads, read back from there
      if (prow) {
        float w[8][kPrepMaxW];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(ptap_s + (pc0 + e) * kPrepMaxW);
#pragma unroll
          for (int i = 0; i < kPrepMaxW; ++i) w[e][i] = t4[i];
        }
        prep_with_window(p.W, [&](auto wc) {
          constexpr int WW = decltype(wc)::value;
#pragma unroll
          for (int r = 0; r < S::RPG; ++r) {
            float x8[kPrepMaxW][8], y[8];
#pragma unroll
            for (int m = kPrepMaxW - WW; m < kPrepMaxW; ++m)
              prep_unpack8(prep_zero_row(cur.kr[r + m], p.k_hist, p.W, c * C + pj0 - (kPrepMaxW - 1) + r + m),
                           x8[m]);
            const float sc = prep_scale(group_sum<S::LPR>(prep_conv8_pad<WW>(w, x8, y)), p.inv_eps);
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (__bf16)(y[e] * sc);
            *reinterpret_cast<bf16x8*>(prow_s + (pj0 + r) * S::PSS + pc0) = o;
          }
        });
      }
      __syncthreads();
      Piece<BF16> xk[S::PPX], kk[S::PPK];
#pragma unroll
      for (int q = 0; q < S::PPX; ++q) {
        const int pc = min(tid + q * S::THREADS, S::NPX - 1);
        const int jp = pc % (CP / 2), c8 = pc / (CP / 2);
        xk[q].a = *reinterpret_cast<const u16x8*>(prow_s + (2 * jp) * S::PSS + 8 * c8);
        xk[q].b = *reinterpret_cast<const u16x8*>(prow_s + (2 * jp + 1) * S::PSS + 8 * c8);
      }
#pragma unroll
      for (int q = 0; q < S::PPK; ++q) {
        const int pc = min(tid + q * S::THREADS, S::NPK - 1);
        const int jp = pc % (CP / 2), c8 = pc / (CP / 2);
        const int col = (FULL ? 0 : 16 * mpart) + 8 * c8;
        kk[q].a = *reinterpret_cast<const u16x8*>(prow_s + (2 * jp) * S::PSS + col);
        kk[q].b = *reinterpret_cast<const u16x8*>(prow_s + (2 * jp + 1) * S::PSS + col);
      }
      if (which == 0) stage_bf16(xk, kk);
      else stage_bf16(cur.x, kk);
    } else if constexpr (BF16) {
      stage_bf16(cur.x, cur.k);
    } else {
      float* Ks = reinterpret_cast<float*>(lds_a);    // [CP][MROWS]
      float* Xs = reinterpret_cast<float*>(lds_b);    // [CP][D] = w_j * X[j][n]
#pragma unroll
      for (int q = 0; q < S::PPX; ++q) {
        const int pc = tid + q * S::THREADS;
        const int j = pc / (D / 4), c4 = pc % (D / 4);
        const float w = __shfl(wj, j & 63, 64);
        if (S::NPX % S::THREADS != 0 && pc >= S::NPX) continue;
        *reinterpret_cast<f32x4*>(Xs + j * D + 4 * c4) = cur.x[q].a * w;
      }
#pragma unroll
      for (int q = 0; q < S::PPK; ++q) {
        const int pc = tid + q * S::THREADS;
        if (S::NPK % S::THREADS != 0 && pc >= S::NPK) continue;
        const int j = pc / (MROWS / 4), c4 = pc % (MROWS / 4);
        *reinterpret_cast<f32x4*>(Ks + j * MROWS + 4 * c4) = cur.k[q].a;
      }
    }
    __syncthreads();

    // ---- delta tiles and state update --------------------------------------------
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
      const int u = wave + S::WAVES * ui;
      if (!S::EVEN && u >= S::NU) continue;
      const int nt = unit_nt(u);
#pragma unroll
      for (int h = 0; h < TPU; ++h) {
        const int mt = unit_mt(u, h);
        const int mrow = FULL ? 16 * mt : 0;   // row offset inside the owned A rows
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (BF16) {
          const __bf16* KT = reinterpret_cast<const __bf16*>(lds_a);
          const __bf16* XH = reinterpret_cast<const __bf16*>(lds_b);
          const __bf16* XL = XH + D * AS;
#pragma unroll
          for (int kb = 0; kb < CP / 32; ++kb) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(KT + (mrow + tl) * AS + 32 * kb + 8 * g);
            const bf16x8 bh_ = *reinterpret_cast<const bf16x8*>(XH + (16 * nt + tl) * AS + 32 * kb + 8 * g);
            const bf16x8 bl_ = *reinterpret_cast<const bf16x8*>(XL + (16 * nt + tl) * AS + 32 * kb + 8 * g);
            acc = mfma_bf16(a, bh_, acc);
            acc = mfma_bf16(a, bl_, acc);
          }
        } else {
          const float* Ks = reinterpret_cast<const float*>(lds_a);
          const float* Xs = reinterpret_cast<const float*>(lds_b);
#pragma unroll 4
          for (int kb = 0; kb < C / 4; ++kb)
            acc = mfma_f32(Ks[(4 * kb + g) * MROWS + mrow + tl], Xs[(4 * kb + g) * D + 16 * nt + tl], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) st[ui][h][i] = gamma_c * st[ui][h][i] + acc[i];
      }
    }
    // whole or segment states: the state before chunk c+1 goes out now, so its
    // stores drain while the next chunk is fetched, gated and staged (measured
    // about 20 % faster than storing it at the top of the next step, at 128
    // sequences of 64 chunks; the stripe walks are not faster this way)
    if constexpr (FULL)
      if (c + 1 < ce) store_snapshot(c + 1);
  };
  if constexpr (DEPTH == 3) {
    for (int c = cb; c < ce; c += 3) {
      step(c, b0, b1, b2);
      if (c + 1 < ce) step(c + 1, b1, b2, b0);
      if (c + 2 < ce) step(c + 2, b2, b0, b1);
    }
  } else {
    for (int c = cb; c < ce; c += 2) {
      step(c, b0, b1, b1);
      if (c + 1 < ce) step(c + 1, b1, b0, b0);
    }
  }

  // ---- final state (fp32, row-major): the sequence's, or a segment total ----------
  float* fin;
  size_t fin_off;
  if constexpr (TOTALS) {
    fin = p.seg_state;
    fin_off = (((size_t)bh * 2 + which) * (p.NS - 1) + seg) * D * D;
    if (which == 0 && u0 == 0 && tid == 0) p.seg_decay[(size_t)bh * (p.NS - 1) + seg] = expf(seg_log);
  } else {
    fin = seg == p.NS - 1 ? (which ? p.g_final : p.h_final) : nullptr;
    fin_off = (size_t)bh * D * D;
  }
  if (fin) {
    float* base = fin + fin_off;
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
      const int u = wave + S::WAVES * ui;
      if (!S::EVEN && u >= S::NU) continue;
      const int nt = unit_nt(u);
#pragma unroll
      for (int h = 0; h < TPU; ++h) {
        const int mt = unit_mt(u, h);
        if (which == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) base[(size_t)(16 * mt + 4 * g + i) * D + 16 * nt + tl] = st[ui][h][i];
        } else {
          *reinterpret_cast<f32x4*>(base + (size_t)(16 * nt + tl) * D + 16 * mt + 4 * g) = st[ui][h];
        }
      }
    }
  }
}

// Carry pass of a segmented walk: for every state entry, fold the segment
// totals in order, C_{s+1} = Gamma_s C_s + total_s (C_0 = h0 / g0 or 0), and
// leave the carry-in state of segment s+1 where total_s was.
__global__ __launch_bounds__(256) void scan_carry_kernel(ScanParams p, int D2) {
  const int q4 = D2 / 4;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)p.BH * 2 * q4) return;
  const int e = (int)(idx % q4);
  const int which = (int)((idx / q4) % 2);
  const int bh = (int)(idx / q4 / 2);
  const float* init = which ? p.g0 : p.h0;
  f32x4 c = init ? *reinterpret_cast<const f32x4*>(init + (size_t)bh * D2 + 4 * e) : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sg = 0; sg < p.NS - 1; ++sg) {
    f32x4* t = reinterpret_cast<f32x4*>(p.seg_state + (((size_t)bh * 2 + which) * (p.NS - 1) + sg) * D2) + e;
    c = p.seg_decay[(size_t)bh * (p.NS - 1) + sg] * c + *t;
    *t = c;
  }
}

template <bool BF16, int D, int C, bool FULL, bool TOTALS>
hipError_t launch_scan_t(const ScanParams& p, hipStream_t s) {
  constexpr int U = ScanShape<BF16, D, C, FULL>::U;
  const int groups = (p.BH + 7) / 8;
  const int nsp = TOTALS ? p.NS - 1 : p.NS;
  const dim3 grid(groups * 8 * U * nsp);
  if constexpr (BF16 && C == 64 && (D == 64 || D == 128)) {
    if (p.prep) {
      hipLaunchKernelGGL((scan_kernel<BF16, D, C, FULL, TOTALS, true>), grid,
                         dim3(ScanShape<BF16, D, C, FULL>::THREADS), 0, s, p);
      return hipGetLastError();
    }
  } else {
    if (p.prep) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((scan_kernel<BF16, D, C, FULL, TOTALS>), grid, dim3(ScanShape<BF16, D, C, FULL>::THREADS), 0, s, p);
  return hipGetLastError();
}

template <bool BF16, int D, int C>
hipError_t launch_scan_c(const ScanParams& p, hipStream_t s) {
  // A whole state per workgroup when there are enough (b, h) slices to give
  // every CU work, or when a long sequence is walked in segments (totals,
  // carry, then the walk proper); otherwise one 16-row stripe per workgroup.
  if (!scan_whole_state(p.BH, p.NC, D)) return launch_scan_t<BF16, D, C, false, false>(p, s);
  if (p.NS > 1) {
    hipError_t e = launch_scan_t<BF16, D, C, true, true>(p, s);
    if (e != hipSuccess) return e;
    const long long n = (long long)p.BH * 2 * (D * D / 4);
    hipLaunchKernelGGL(scan_carry_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, D * D);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_scan_t<BF16, D, C, true, false>(p, s);
}

template <bool BF16, int D>
hipError_t launch_scan_d(int C, const ScanParams& p, hipStream_t s) {
  switch (C) {
    case 16: return launch_scan_c<BF16, D, 16>(p, s);
    case 32: return launch_scan_c<BF16, D, 32>(p, s);
    case 64: return launch_scan_c<BF16, D, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan(bool bf16, int D, int C, const ScanParams& p, hipStream_t s) {
  if (bf16) {
    switch (D) {
      case 32: return launch_scan_d<true, 32>(C, p, s);
      case 64: return launch_scan_d<true, 64>(C, p, s);
      case 128: return launch_scan_d<true, 128>(C, p, s);
    }
  } else {
    switch (D) {
      case 16: return launch_scan_d<false, 16>(C, p, s);
      case 32: return launch_scan_d<false, 32>(C, p, s);
      case 64: return launch_scan_d<false, 64>(C, p, s);
      case 128: return launch_scan_d<false, 128>(C, p, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace mesa
