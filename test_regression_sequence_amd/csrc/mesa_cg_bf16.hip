// Chunked CG solve + read-out, bf16 inputs (MFMA bf16, fp32 accumulation).
//
// Same mathematics as the generic kernel in mesa_cg.hip (MesaNet page,
// technical summary, "Mesa layer": CG query response, chunk-parallel states,
// dynamic CG step count); this file is the tuned bf16 path.
//
// Within a chunk of tokens s..e with b_t = sum_{i=s..t} log gamma_i and
// Gamma_t = e^{b_t}, the system of token t is
//     A_t = Gamma_t Hb + sum_{j<=t} e^{b_t - b_j} beta_j k_j k_j^T + Lambda.
// Divided by Gamma_t it becomes
//     A_t / Gamma_t = Hb + sum_{j<=t} w_j k_j k_j^T + Lambda / Gamma_t,
//     w_j = beta_j e^{-b_j},
// whose key weights no longer depend on t.  CG on (A_t / Gamma_t) xh = q from
// xh = 0 has exactly the residuals, search directions and step counts of CG
// on A_t x = q, with xh = Gamma_t x; and the output needs no rescaling:
//     o_t = G_t x = Gb xh + sum_{j<=t} w_j (k_j . xh) v_j.
// So the weights fold into the key (value) columns once per chunk, the
// boundary-state product needs no per-token multiply, and the causal mask is
// all that is left per iteration.  A chunk that decays so strongly that
// e^{-b_j} could overflow (e^{-b_e} > e^40) is only flagged here; the kernel
// in mesa_cg_bf16_unscaled.hip then solves it in the unscaled form.
//
// One wave per chunk.  The wave loads the chunk's boundary state and keys
// once, then runs the CG of its NW = C/16 token tiles one after another (each
// tile leaves its loop as soon as its 16 tokens have stopped), parks every
// tile's solution in LDS, and finally loads Gb and the values once for the
// read-out of all tiles.  Every tile has its own straight-line code (the
// causal extent of a tile is a compile-time constant).  A grid with fewer
// chunks than SIMDs shares each chunk out over 2 or 4 waves instead (tiles
// {0, 3} and {1, 2}, or one tile each): every wave loads the chunk's operands
// itself and solves and reads out only its tiles, with the same arithmetic
// per tile, so the results are bitwise those of one wave per chunk.
//
// Register layout (lane l, tl = l%16, g = l/16): every CG vector of token
// 16w + tl keeps dims 16a + 4g + {0..3} (a < D/16) as f32x4 v[a].  Matrix
// products are MFMA 16x16x32 bf16 with the per-token vectors as the B
// operand; the contraction index of each MFMA is permuted so that register
// pairs (v[2m], v[2m+1]) form the B operand of k-block m directly.
//
// Every A operand the CG loop needs is loop-invariant and lives in the
// accumulation registers (AGPRs), which MFMA reads directly:
//   mf[nt][m]   boundary state Hb (Gb for the read-out), fragment order as
//               written by the scan kernel: row 16nt+tl, cols 32m+4g+{0..3},
//               32m+16+4g+{0..3};
//   kr[jt][m]   key rows:    K[16jt+tl][32m+4g+{0..3}, 32m+16+4g+{0..3}];
//   kc[nt][mj]  weighted key columns: w_j K[j][16nt+tl] for
//               j = 32mj+4g+{0..3}, 32mj+16+4g+{0..3} (weighted value
//               columns for the read-out).
// The state and the row fragments are fetched from global memory in one
// batch; the column fragments are then formed from the (weighted) row
// fragments by an exact MFMA transpose, so the CG loop touches no global
// memory.  MFMA accumulators stay in VGPRs (built with -amdgpu-mfma-vgpr-form).
//
// WARM (warm-started CG; the "significance" section names warm-started
// optimisation as a way to cut the solver's cost): tile w >= 1 starts each
// token t from token t-16's solution, which the same lane of the same wave
// produced in tile w-1, rescaled to the scaled form, xh_0 = e^{b_t - b_{t-16}}
// xh_{t-16}, with r_0 = q - (A_t / Gamma_t) xh_0 from one more product (not
// counted as a step).  Tile 0 starts from 0: earlier chunks are solved in
// parallel.
//
// PREP (fused preprocessing, the "architecture" section: queries and keys
// are convolved with a small causal window and normalised before the layer):
// q and k arrive raw; the wave forms the chunk's processed keys, then its
// processed queries, into one LDS buffer (mesa_prep_rows.h, the same
// arithmetic as the preprocessing kernel) and reads the key row fragments and
// each tile's queries from there instead of from global memory.
//
// Lambda is diagonal, or (LF) a full symmetric positive definite matrix per
// head (the page calls the regulariser symmetric positive definite).  The
// full matrix enters as one more d x d MFMA operand, (Lambda / Gamma_t) p =
// Lambda (e^{-b_t} p): its bf16 fragments sit in LDS, since the AGPRs already
// hold Hb and the keys, and the B operand is the search direction scaled per
// token.  Two chunks of one sequence share a workgroup (one wave each) and one
// copy of Lambda, so that four waves still fit a CU's LDS.
#include <atomic>
#include <type_traits>

#include "mesa_common.h"
#include "mesa_kernels.h"
#include "mesa_prep_rows.h"

namespace mesa {

namespace {

template <int W>
using tile_c = std::integral_constant<int, W>;

// LDS of one workgroup (declared once per kernel; the bodies below take it by reference)
template <int D, int C, bool LF, bool PREP>
struct CgLds {
  static constexpr int ND = D / 16, NM = ND / 2, NW = C / 16, NWV = LF ? 2 : 1;
  static constexpr int PS = D + 8;  // PREP row stride, padded by 16 bytes against bank conflicts
  bf16x8 xs_[NWV][NW * NM * 64];    // solutions xh of the tiles as bf16, [tile][m][lane]
  bf16x8 lamf[LF ? ND * NM * 64 : 1];  // full Lambda as A fragments, [nt][m][lane]
  float lam_s[D];
  float bcum_[NWV][C];
  float betas_[NWV][C];
  // PREP: the chunk's processed keys, then its processed queries, [row][D]
  __attribute__((aligned(16))) __bf16 prow[PREP ? C * PS : 1];
};

// One wave's work on one chunk.  SP waves share a chunk's token tiles (SP = 1:
// all of them); PART is this wave's share, known at compile time so that each
// share is straight-line code of its own.
template <int D, int C, bool LF, bool WARM, bool PREP, int SP, int PART>
__device__ __forceinline__ void cg_chunk(const CgParams& p, CgLds<D, C, LF, PREP>& L) {
  static_assert(!(LF && WARM), "the warm start takes a diagonal Lambda");
  static_assert(!PREP || (!LF && !WARM && C == 64), "fused preprocessing: diagonal Lambda, cold start, chunk 64");
  static_assert(SP == 1 || (!LF && !WARM && !PREP && (SP == 2 || SP == 4) && SP <= C / 16),
                "shared chunks: the plain kernel, 2 or 4 waves per chunk, at most one per tile");
  constexpr int ND = D / 16, NM = ND / 2, NW = C / 16, NMJ = (NW + 1) / 2;
  constexpr int NWV = LF ? 2 : 1;  // waves (chunks) per workgroup

  const int lane = threadIdx.x & 63, tl = lane & 15, g = lane >> 4;
  const int wv = NWV > 1 ? (int)(threadIdx.x >> 6) : 0;
  int bh, c;
  if constexpr (NWV > 1) {
    // chunks 2i and 2i+1 of sequence bh; past an odd chunk count the second
    // wave only helps to stage Lambda (its loads repeat the last chunk's)
    const int ncp = (p.NC + 1) / 2;
    bh = blockIdx.x / ncp;
    c = 2 * (blockIdx.x % ncp) + wv;
  } else {
    const int blk = SP > 1 ? (int)(blockIdx.x / SP) : (int)blockIdx.x;
    bh = blk / p.NC;
    c = blk % p.NC;
  }
  const bool has_chunk = c < p.NC;
  if (!has_chunk) c = p.NC - 1;
  const int chunk = bh * p.NC + c;
  const int h = bh % p.H;
  const int T = p.T, s = c * C, Lc = min(C, T - s);
  const size_t row0 = (size_t)bh * T + s;

  auto& xs_ = L.xs_;
  auto& lamf = L.lamf;
  auto& lam_s = L.lam_s;
  auto& bcum_ = L.bcum_;
  auto& betas_ = L.betas_;
  constexpr int PS = CgLds<D, C, LF, PREP>::PS;
  auto& prow = L.prow;
  bf16x8* const xs = xs_[wv];
  float* const bcum = bcum_[wv];
  float* const betas = betas_[wv];

  const uint16_t* Kg = static_cast<const uint16_t*>(p.k);
  const uint16_t* Vg = static_cast<const uint16_t*>(p.v);
  const uint16_t* Qg = static_cast<const uint16_t*>(p.q);
  const size_t snap = (size_t)chunk * (D * D / 8);

  // ---- one batch of loads: state, key rows, gates, Lambda ----------------------
  bf16x8 mf[ND][NM];
  bf16x8 kr[NW][NM];
  bf16x8 kc[ND][NMJ];
  auto load_state = [&](const void* base) {
    const bf16x8* F = static_cast<const bf16x8*>(base) + snap;
#pragma unroll
    for (int nt = 0; nt < ND; ++nt)
#pragma unroll
      for (int m = 0; m < NM; ++m) mf[nt][m] = F[(nt * NM + m) * 64 + lane];
  };
  // row fragments X[16jt+tl][32m+4g+{0..3}, 32m+16+4g+{0..3}].  Rows past Lc
  // (a ragged last chunk) repeat row Lc-1: their weight w_j is 0, so their
  // weighted columns are zero and they contribute nothing.  Every load is
  // unconditional, so the whole batch is in flight at once.
  auto load_rows = [&](const uint16_t* X, bf16x8 (&dst)[NW][NM]) {
#pragma unroll
    for (int jt = 0; jt < NW; ++jt) {
      const int j = min(16 * jt + tl, Lc - 1);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint16_t* src = X + (row0 + j) * D + 32 * m + 4 * g;
        const u16x4 lo = *reinterpret_cast<const u16x4*>(src);
        const u16x4 hi = *reinterpret_cast<const u16x4*>(src + 16);
        dst[jt][m] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  // PREP: the key row fragments from the processed rows in LDS (rows past Lc
  // hold finite filler, weighted 0 like the repeated rows above)
  auto load_rows_lds = [&](bf16x8 (&dst)[NW][NM]) {
#pragma unroll
    for (int jt = 0; jt < NW; ++jt)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const __bf16* src = prow + (16 * jt + tl) * PS + 32 * m + 4 * g;
        const u16x4 lo = *reinterpret_cast<const u16x4*>(src);
        const u16x4 hi = *reinterpret_cast<const u16x4*>(src + 16);
        dst[jt][m] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
  };
  // Column fragments from row fragments, transposed on the MFMA unit: with B
  // the 0/1 matrix selecting dims 16nt..16nt+15 out of k-block nt/2, the
  // product's lane (tl, g) holds X[16jt+4g+i][16nt+tl] (exact: one nonzero
  // bf16 x 1.0 term per sum, and the value is bf16 again).
  bf16x8 sel[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    u16x8 v = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if ((tl >> 2) == g) v[4 * par + (tl & 3)] = 0x3F80;  // bf16 1.0
    sel[par] = __builtin_bit_cast(bf16x8, v);
  }
  auto columns_from_rows = [&](const bf16x8 (&rows)[NW][NM]) {
#pragma unroll
    for (int mj = 0; mj < NMJ; ++mj) {
#pragma unroll
      for (int nt = 0; nt < ND; ++nt) {
        const int jl = 2 * mj, jh = (2 * mj + 1) % NW;
        const f32x4 lo = mfma_bf16(rows[jl][nt >> 1], sel[nt & 1], f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 hi = (2 * mj + 1 < NW) ? mfma_bf16(rows[jh][nt >> 1], sel[nt & 1], f32x4{0.f, 0.f, 0.f, 0.f})
                                           : f32x4{0.f, 0.f, 0.f, 0.f};
        kc[nt][mj] = pack8(lo, hi);
      }
    }
  };
  // rows times the per-row key weight w_{16jt+tl} (scaled form), rounded to bf16
  auto weighted_rows = [&](const bf16x8 (&rows)[NW][NM], bf16x8 (&dst)[NW][NM]) {
#pragma unroll
    for (int jt = 0; jt < NW; ++jt) {
      const int j = 16 * jt + tl;
      const float wj = (j < Lc) ? betas[j] * expf(-bcum[j]) : 0.f;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const u16x8 u = __builtin_bit_cast(u16x8, rows[jt][m]);
        f32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = wj * bf16_to_f32(u[e]);
          hi[e] = wj * bf16_to_f32(u[4 + e]);
        }
        dst[jt][m] = pack8(lo, hi);
      }
    }
  };
  // keep the loop-invariant MFMA A operands in accumulation registers
  auto pin_operands = [&]() {
#pragma unroll
    for (int nt = 0; nt < ND; ++nt)
#pragma unroll
      for (int m = 0; m < NM; ++m) asm volatile("" : "+a"(mf[nt][m]));
#pragma unroll
    for (int jt = 0; jt < NW; ++jt)
#pragma unroll
      for (int m = 0; m < NM; ++m) asm volatile("" : "+a"(kr[jt][m]));
#pragma unroll
    for (int nt = 0; nt < ND; ++nt)
#pragma unroll
      for (int mj = 0; mj < NMJ; ++mj) asm volatile("" : "+a"(kc[nt][mj]));
  };

  // queries of one tile as raw bf16 (tokens past Lc read row Lc-1 and are
  // zeroed when converted); the next tile's are fetched while the current
  // tile iterates
  u16x4 qraw[ND];
  auto fetch_q = [&](const int w) {
    const int tq = min(16 * w + tl, Lc - 1);
#pragma unroll
    for (int a = 0; a < ND; ++a) {
      if constexpr (PREP) qraw[a] = *reinterpret_cast<const u16x4*>(prow + (16 * w + tl) * PS + 16 * a + 4 * g);
      else qraw[a] = *reinterpret_cast<const u16x4*>(Qg + (row0 + tq) * D + 16 * a + 4 * g);
    }
  };
  // PREP: the raw rows of the chunk's keys and queries, loaded in the first
  // batch and formed into prow one after the other
  PrepChunk<D, C> kraw, qraw_rows;
  auto prep_load = [&](PrepChunk<D, C>& pc, const void* X, const void* hist) {
    pc.load(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(hist), bh, T, p.W, s, Lc, lane);
  };
  auto prep_form = [&](const PrepChunk<D, C>& pc, const float* taps) {
    pc.form(taps, h, p.W, p.inv_eps, prow, PS, lane);
  };

  if constexpr (LF) {
    // Lambda[16nt+tl][32m+4g+{0..3}, 32m+16+4g+{0..3}] of the head, rounded to
    // bf16; the two waves stage alternate fragments (the barrier below
    // publishes them), and a lane reads only its own slots
    const float* L = p.lam + (size_t)h * D * D;
#pragma unroll 4
    for (int f = wv; f < ND * NM; f += NWV) {
      const int nt = f / NM, m = f % NM;
      const float* src = L + (size_t)(16 * nt + tl) * D + 32 * m + 4 * g;
      lamf[f * 64 + lane] = pack8(*reinterpret_cast<const f32x4*>(src), *reinterpret_cast<const f32x4*>(src + 16));
    }
  }
  // gates first: their prefix scan overlaps the state and key loads
  {
    float lg = 0.f, bt = 0.f;
    float lam_v[(D + 63) / 64];
    if (lane < Lc) {
      lg = p.gamma[row0 + lane];
      bt = p.beta[row0 + lane];
    }
#pragma unroll
    for (int i = 0; i < (D + 63) / 64; ++i)
      lam_v[i] = (!LF && lane + 64 * i < D) ? p.lam[(size_t)h * D + lane + 64 * i] : 0.f;
    if constexpr (PREP) {
      prep_load(kraw, p.k, p.k_hist);
      prep_load(qraw_rows, p.q, p.q_hist);
    }
    load_state(p.hb);
    if constexpr (PREP) {
      prep_form(kraw, p.wk);
      __syncthreads();
      load_rows_lds(kr);
    } else {
      load_rows(Kg, kr);
      fetch_q(PART);  // the wave's first tile (PART, in every split)
    }
    lg = lane < Lc ? logf(lg) : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_up(lg, o, 64);
      if (lane >= o) lg += t;
    }
    if (lane < C) {
      bcum[lane] = lg;
      betas[lane] = bt;
    }
#pragma unroll
    for (int i = 0; i < (D + 63) / 64; ++i)
      if (lane + 64 * i < D) lam_s[lane + 64 * i] = lam_v[i];
  }
  __syncthreads();
  if (!has_chunk) return;
  // the chunk's total decay decides the form (wave-uniform); a chunk left to
  // the unscaled kernel is flagged for it
  const bool scaled = __builtin_amdgcn_readfirstlane(bcum[Lc - 1] >= -kMaxScaledDecay ? 1 : 0) != 0;
  if (lane == 0) p.unscaled[chunk] = scaled ? 0 : 1;
  if (!scaled) return;
  if constexpr (PREP) {
    // the key fragments are in registers (the barrier above waited for them):
    // the queries replace the keys in the buffer
    prep_form(qraw_rows, p.wq);
    __syncthreads();
    fetch_q(0);
  }
  {
    bf16x8 wr[NW][NM];
    weighted_rows(kr, wr);
    columns_from_rows(wr);
  }
  pin_operands();

  // ---- per-tile machinery ----------------------------------------------------------

  // The causal part of a tile's product: with the score tiles sc[jt] of its
  // tokens against key tile jt (jt <= w), mask the diagonal block (j <= t),
  // pack the scores to bf16 and add Y^T S^T to acc[nt] (the key weights sit in
  // the key columns).
  f32x4 acc[ND];
  auto add_intra = [&](auto wc, f32x4* sc) {
    constexpr int w = decltype(wc)::value;
#pragma unroll
    for (int jt = 0; jt <= w; ++jt) asm volatile("" : "+v"(sc[jt]));
    bf16x8 sb[w / 2 + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[w][i] = (4 * g + i <= tl) ? sc[w][i] : 0.f;
#pragma unroll
    for (int mj = 0; mj <= w / 2; ++mj) {
      const f32x4 hi = (2 * mj + 1 <= w) ? sc[2 * mj + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
      sb[mj] = pack8(sc[2 * mj], hi);
    }
#pragma unroll
    for (int mj = 0; mj <= w / 2; ++mj)
#pragma unroll
      for (int nt = 0; nt < ND; ++nt) acc[nt] = mfma_bf16(kc[nt][mj], sb[mj], acc[nt]);
  };
  // acc[nt] <- Mb u + Y^T S^T for a bf16 vector u given as k-blocks ub (the
  // read-out): score MFMAs, boundary-state MFMAs, then the masked scores'
  // MFMAs, so no instruction waits on an MFMA issued just before it
  auto matvec = [&](auto wc, const bf16x8* ub) {
    constexpr int w = decltype(wc)::value;
    f32x4 sc[w + 1];
#pragma unroll
    for (int jt = 0; jt <= w; ++jt) {
      sc[jt] = mfma_bf16(kr[jt][0], ub[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int m = 1; m < NM; ++m) sc[jt] = mfma_bf16(kr[jt][m], ub[m], sc[jt]);
    }
#pragma unroll
    for (int nt = 0; nt < ND; ++nt) {
      acc[nt] = mfma_bf16(mf[nt][0], ub[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int m = 1; m < NM; ++m) acc[nt] = mfma_bf16(mf[nt][m], ub[m], acc[nt]);
    }
    add_intra(wc, sc);
#pragma unroll
    for (int nt = 0; nt < ND; ++nt) asm volatile("" : "+v"(acc[nt]));
  };

  // ---- conjugate gradient of one tile -------------------------------------------
  f32x4 xprev[WARM ? ND : 1];  // the previous tile's solutions (WARM)
  auto solve_tile = [&](auto wc, auto nc) {
    constexpr int w = decltype(wc)::value;
    const int tloc = 16 * w + tl;
    const bool valid = tloc < Lc;
    // 1 / Gamma_t of the lane's token, and Lambda / Gamma_t for a diagonal
    // Lambda, held for the whole loop
    const float lscale = expf(-bcum[tloc]);
    f32x4 lt[LF ? 1 : ND];
    if constexpr (!LF) {
#pragma unroll
      for (int a = 0; a < ND; ++a) lt[a] = *reinterpret_cast<const f32x4*>(&lam_s[16 * a + 4 * g]) * lscale;
    }
    f32x4 r[ND], x[ND], pv[ND];
#pragma unroll
    for (int a = 0; a < ND; ++a) {
      r[a] = valid ? f32x4{bf16_to_f32(qraw[a][0]), bf16_to_f32(qraw[a][1]), bf16_to_f32(qraw[a][2]),
                           bf16_to_f32(qraw[a][3])}
                   : f32x4{0.f, 0.f, 0.f, 0.f};
      x[a] = f32x4{0.f, 0.f, 0.f, 0.f};
      pv[a] = r[a];
    }
    if constexpr (WARM && w > 0) {
      // xh_0 = e^{b_t - b_{t-16}} xh_{t-16}; r_0 = q - (A_t / Gamma_t) xh_0
      const float sh = valid ? expf(bcum[tloc] - bcum[tloc - 16]) : 0.f;
      bf16x8 ub[NM];
#pragma unroll
      for (int a = 0; a < ND; ++a) x[a] = xprev[a] * sh;
#pragma unroll
      for (int m = 0; m < NM; ++m) ub[m] = pack8(x[2 * m], x[2 * m + 1]);
      pin_operands();
      matvec(wc, ub);
#pragma unroll
      for (int a = 0; a < ND; ++a) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[a][i] -= __builtin_fmaf(lt[a][i], x[a][i], acc[a][i]);
        pv[a] = r[a];
      }
    }
    if constexpr (decltype(nc)::value >= 0) fetch_q(decltype(nc)::value);  // the wave's next tile
    float rho = 0.f;
#pragma unroll
    for (int a = 0; a < ND; ++a) rho += r[a][0] * r[a][0] + r[a][1] * r[a][1] + r[a][2] * r[a][2] + r[a][3] * r[a][3];
    rho = sum_lane_groups(rho);
    int n = 0;
    bool stopped = false;
    // the previous step's alpha and beta: its x step and the new direction are
    // formed block by block at the top of the next iteration, among its MFMAs
    float alpha_p = 0.f, beta_p = 0.f;
    // the loop runs while some token of the tile is active (one test, at the
    // bottom, from the state the step left)
    bool active = rho >= kCgZero && rho > p.tol2;
    int it = 0;
    if (p.max_steps > 0 && __any(active)) do {
      pin_operands();
      // per k-block m (the dims of pv[2m], pv[2m+1]): x += alpha_p p, then
      // p = r + beta_p p in place (three-operand FMA: the two-address form would
      // tie the result to r, which stays live), its bf16 copy, and every MFMA
      // that reads that copy -- so block m+1's vector work issues while block
      // m's MFMAs run
      f32x4 sc[w + 1];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int a = 2 * m + hh;
          x[a] += alpha_p * pv[a];
#pragma unroll
          for (int i = 0; i < 4; ++i) asm("v_fma_f32 %0, %1, %0, %2" : "+v"(pv[a][i]) : "v"(beta_p), "v"(r[a][i]));
        }
        const bf16x8 ub = pack8(pv[2 * m], pv[2 * m + 1]);
#pragma unroll
        for (int jt = 0; jt <= w; ++jt) sc[jt] = mfma_bf16(kr[jt][m], ub, m == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sc[jt]);
#pragma unroll
        for (int nt = 0; nt < ND; ++nt) acc[nt] = mfma_bf16(mf[nt][m], ub, m == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[nt]);
        if constexpr (LF) {
          // + Lambda (e^{-b_t} p) over the dims of block m
          const bf16x8 us = pack8(pv[2 * m] * lscale, pv[2 * m + 1] * lscale);
#pragma unroll
          for (int nt = 0; nt < ND; ++nt) acc[nt] = mfma_bf16(lamf[(nt * NM + m) * 64 + lane], us, acc[nt]);
        }
      }
      add_intra(wc, sc);
      // + (Lambda / Gamma_t) p for a diagonal Lambda, then w = acc and p.w (two
      // independent chains)
      float pw0 = 0.f, pw1 = 0.f;
#pragma unroll
      for (int a = 0; a < ND; ++a) {
        if constexpr (!LF) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[a][i] = __builtin_fmaf(lt[a][i], pv[a][i], acc[a][i]);
        }
        pw0 += pv[a][0] * acc[a][0];
        pw1 += pv[a][1] * acc[a][1];
        pw0 += pv[a][2] * acc[a][2];
        pw1 += pv[a][3] * acc[a][3];
      }
      const float pw = sum_lane_groups(pw0 + pw1);
      const bool ok = active && pw >= kCgZero;
      stopped = !ok;
      const float alpha = ok ? rho * __builtin_amdgcn_rcpf(pw) : 0.f;
      float rr0 = 0.f, rr1 = 0.f;
#pragma unroll
      for (int a = 0; a < ND; ++a) {
        r[a] -= alpha * acc[a];
        rr0 += r[a][0] * r[a][0];
        rr1 += r[a][1] * r[a][1];
        rr0 += r[a][2] * r[a][2];
        rr1 += r[a][3] * r[a][3];
      }
      const float rr = sum_lane_groups(rr0 + rr1);
      // a stopped token keeps x and r (alpha = 0); its direction becomes r,
      // which stays finite and is never used again
      const float bet = ok ? rr * __builtin_amdgcn_rcpf(rho) : 0.f;
      alpha_p = alpha;
      beta_p = bet;
      rho = ok ? rr : rho;
      n += ok ? 1 : 0;
      active = !stopped && rho >= kCgZero && rho > p.tol2;
    } while (++it < p.max_steps && __any(active));
    // the last step's x update
#pragma unroll
    for (int a = 0; a < ND; ++a) x[a] += alpha_p * pv[a];
    if constexpr (WARM) {
#pragma unroll
      for (int a = 0; a < ND; ++a) xprev[a] = x[a];
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) xs[(w * NM + m) * 64 + lane] = pack8(x[2 * m], x[2 * m + 1]);
    if (valid) {
      if (p.x_out) {
        // x = xh / Gamma_t
        const float xscale = expf(-bcum[tloc]);
#pragma unroll
        for (int a = 0; a < ND; ++a)
          *reinterpret_cast<f32x4*>(p.x_out + (row0 + tloc) * D + 16 * a + 4 * g) = x[a] * xscale;
      }
      if (p.steps && g == 0) p.steps[row0 + tloc] = n;
    }
  };

  // ---- read-out of one tile: o_t = Gb xh + sum_{j<=t} w_j (k_j . xh) v_j --------
  auto readout_tile = [&](auto wc) {
    constexpr int w = decltype(wc)::value;
    const int tloc = 16 * w + tl;
    bf16x8 xb[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) xb[m] = xs[(w * NM + m) * 64 + lane];
    pin_operands();
    matvec(wc, xb);
    if (tloc < Lc) {
#pragma unroll
      for (int a = 0; a < ND; ++a)
        *reinterpret_cast<f32x4*>(p.o + (row0 + tloc) * D + 16 * a + 4 * g) = acc[a];
    }
  };

  // The wave's tiles, each with the next one to prefetch (-1: none): all of
  // them in order (SP == 1); tile PART (SP == NW); or, two waves on four
  // tiles, {0, 3} and {1, 2}, which balances their causal extents.
  auto for_tiles = [&](auto fn) {
    using none = tile_c<-1>;
    if constexpr (SP == 1) {
      fn(tile_c<0>{}, tile_c<(NW > 1 ? 1 : -1)>{});
      if constexpr (NW > 1) fn(tile_c<(NW > 1 ? 1 : 0)>{}, tile_c<(NW > 2 ? 2 : -1)>{});
      if constexpr (NW > 2) fn(tile_c<(NW > 2 ? 2 : 0)>{}, tile_c<(NW > 3 ? 3 : -1)>{});
      if constexpr (NW > 3) fn(tile_c<(NW > 3 ? 3 : 0)>{}, none{});
    } else if constexpr (SP == NW) {
      fn(tile_c<PART>{}, none{});
    } else {
      static_assert(SP == 2 && NW == 4, "two waves on four tiles");
      if constexpr (PART == 0) {
        fn(tile_c<0>{}, tile_c<3>{});
        fn(tile_c<3>{}, none{});
      } else {
        fn(tile_c<1>{}, tile_c<2>{});
        fn(tile_c<2>{}, none{});
      }
    }
  };

  for_tiles(solve_tile);
  if (!p.o) return;  // solutions only (the backward's adjoint solves)

  // Gb and the (weighted) value columns replace Hb and the key columns (the
  // key rows stay: the scores of x are against the keys).
  load_state(p.gb);
  {
    bf16x8 vr[NW][NM];
    load_rows(Vg, vr);
    bf16x8 wr[NW][NM];
    weighted_rows(vr, wr);
    columns_from_rows(wr);
  }
  pin_operands();
  for_tiles([&](auto wc, auto) { readout_tile(wc); });
}

template <int D, int C, bool LF, bool WARM = false, bool PREP = false, int SP = 1>
__global__ __launch_bounds__(LF ? 128 : 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void cg_bf16_kernel(CgParams p) {
  __shared__ CgLds<D, C, LF, PREP> lds;
  if constexpr (SP == 1) {
    cg_chunk<D, C, LF, WARM, PREP, 1, 0>(p, lds);
  } else {
    // each share is its own code path from the top (no live range crosses
    // the branch)
    const int part = (int)(blockIdx.x % SP);
    if (part == 0) {
      cg_chunk<D, C, LF, WARM, PREP, SP, 0>(p, lds);
    } else if (part == 1) {
      cg_chunk<D, C, LF, WARM, PREP, SP, 1>(p, lds);
    } else if constexpr (SP == 4) {
      if (part == 2) cg_chunk<D, C, LF, WARM, PREP, SP, 2>(p, lds);
      else cg_chunk<D, C, LF, WARM, PREP, SP, 3>(p, lds);
    }
  }
}

// Compute units of the current device (looked up once per device; calls from
// several host threads may look it up at once and store the same value).
int device_cus() {
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Waves per chunk for the plain kernel.  A grid of fewer chunks than SIMDs
// leaves SIMDs idle while each wave solves its tiles one after another;
// sharing a chunk's tiles out over 2 or 4 waves (each loads the chunk's
// operands itself) puts them to work.  A SIMD that already runs a wave gains
// nothing from a second one: the CG loop keeps its vector unit busy.
template <int C>
int split_waves(long long chunks) {
  constexpr int NW = C / 16;
  const long long simds = 4LL * device_cus();
  if (NW >= 4 && 4 * chunks <= simds) return 4;
  if (NW >= 2 && 2 * chunks <= simds) return 2;
  return 1;
}

template <int D, int C, bool LF = false>
hipError_t launch_t(const CgParams& p, hipStream_t s) {
  // LF: two chunks of one sequence per two-wave workgroup
  const dim3 grid((unsigned)((long long)p.BH * (LF ? (p.NC + 1) / 2 : p.NC)));
  if constexpr (!LF) {
    if (p.prep) {
      if constexpr (C == 64 && D >= 64) {
        if (p.warm) return hipErrorInvalidValue;
        hipLaunchKernelGGL((cg_bf16_kernel<D, C, false, false, true>), grid, dim3(64), 0, s, p);
      } else {
        return hipErrorInvalidValue;
      }
    } else if (p.warm) {
      hipLaunchKernelGGL((cg_bf16_kernel<D, C, false, true>), grid, dim3(64), 0, s, p);
    } else {
      const long long chunks = (long long)p.BH * p.NC;
      const int sp = split_waves<C>(chunks);
      if constexpr (C >= 64) {
        if (sp == 4)
          hipLaunchKernelGGL((cg_bf16_kernel<D, C, false, false, false, 4>), dim3((unsigned)(4 * chunks)), dim3(64),
                             0, s, p);
      }
      if constexpr (C >= 32) {
        if (sp == 2)
          hipLaunchKernelGGL((cg_bf16_kernel<D, C, false, false, false, 2>), dim3((unsigned)(2 * chunks)), dim3(64),
                             0, s, p);
      }
      if (sp == 1) hipLaunchKernelGGL((cg_bf16_kernel<D, C, false, false>), grid, dim3(64), 0, s, p);
    }
  } else {
    if (p.warm || p.prep) return hipErrorInvalidValue;
    hipLaunchKernelGGL((cg_bf16_kernel<D, C, LF>), grid, dim3(128), 0, s, p);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_cg_bf16_unscaled(D, C, p, s);
}

template <int D>
hipError_t launch_d(int C, const CgParams& p, hipStream_t s) {
  switch (C) {
    case 16: return launch_t<D, 16>(p, s);
    case 32: return launch_t<D, 32>(p, s);
    case 64: return launch_t<D, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_cg_bf16(int D, int C, const CgParams& p, hipStream_t s) {
  if (p.lam_full) {
    if (C != 64) return hipErrorInvalidValue;
    if (D == 64) return launch_t<64, 64, true>(p, s);
    if (D == 128) return launch_t<128, 64, true>(p, s);
    return hipErrorInvalidValue;
  }
  switch (D) {
    case 32: return launch_d<32>(C, p, s);
    case 64: return launch_d<64>(C, p, s);
    case 128: return launch_d<128>(C, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mesa
