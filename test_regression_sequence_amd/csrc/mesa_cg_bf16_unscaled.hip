// Chunked CG solve + read-out, bf16 inputs, unscaled form: the chunks whose
// decay is too strong for the scaled kernel in mesa_cg_bf16.hip.
//
// Same mathematics (MesaNet page, technical summary, "Mesa layer": CG query
// response, chunk-parallel states, dynamic CG step count).  Within a chunk,
// with b_t = sum_{i=s..t} log gamma_i and Gamma_t = e^{b_t},
//     (H_t + Lambda) p = Gamma_t Hb p + sum_{j<=t} W_tj (k_j . p) k_j + Lambda p,
//     W_tj = e^{b_t - b_j} beta_j,
// whose factors never exceed 1 whatever the decay, so no scaling can
// overflow.  The scaled kernel flags every chunk it leaves; this kernel reads
// the flags of 8 chunks per wave and solves the flagged ones, so on inputs
// with moderate decay it costs one flag read per wave.
//
// The organisation follows the scaled kernel: one wave per chunk, loop-
// invariant MFMA A operands in AGPRs (boundary state, key rows, key columns
// formed by an exact MFMA transpose), CG of the NW = C/16 token tiles one
// after another, solutions parked in LDS, read-out with Gb and value columns.
// Register layout (lane l, tl = l%16, g = l/16): CG vectors of token 16w + tl
// keep dims 16a + 4g + {0..3} as f32x4 v[a].  A full symmetric positive
// definite Lambda (LF) enters as one more MFMA operand, its bf16 fragments in
// LDS, applied to the bf16 search direction.  WARM: tile w >= 1 starts token t
// from token t-16's solution (the previous tile's, parked in LDS), with
// r_0 = q - A_t x_0 from one more product, as in the scaled kernel.  PREP:
// q and k arrive raw and are convolved and normalised into LDS as they are
// loaded, as in the scaled kernel.
#include "mesa_common.h"
#include "mesa_kernels.h"
#include "mesa_prep_rows.h"

namespace mesa {

namespace {

constexpr int kChunksPerWave = 8;

template <int D, int C, bool LF, bool WARM = false, bool PREP = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void cg_bf16_unscaled_kernel(CgParams p) {
  static_assert(!(LF && WARM), "the warm start takes a diagonal Lambda");
  static_assert(!PREP || (!LF && !WARM && C == 64), "fused preprocessing: diagonal Lambda, cold start, chunk 64");
  constexpr int ND = D / 16, NM = ND / 2, NW = C / 16, NMJ = (NW + 1) / 2;

  const int lane = threadIdx.x, tl = lane & 15, g = lane >> 4;
  const int nchunks = p.BH * p.NC;
  const int first = blockIdx.x * kChunksPerWave;
  const bool flagged = lane < kChunksPerWave && first + lane < nchunks && p.unscaled[first + lane] != 0;
  uint64_t todo = __ballot(flagged);

  __shared__ f32x4 xs[NW * ND * 64];   // solutions of the tiles, [tile][a][lane]
  __shared__ float lam_s[D];
  __shared__ bf16x8 lamf[LF ? ND * NM * 64 : 1];  // full Lambda as A fragments, [nt][m][lane]
  __shared__ float bcum[C];
  __shared__ float betas[C];
  // PREP: the chunk's processed keys, then its processed queries, [row][D]
  constexpr int PS = D + 8;
  __shared__ __attribute__((aligned(16))) __bf16 prow[PREP ? C * PS : 1];

  while (todo) {
    const int chunk = first + __builtin_ctzll(todo);
    todo &= todo - 1;
    const int bh = chunk / p.NC, c = chunk % p.NC;
    const int h = bh % p.H;
    const int T = p.T, s = c * C, Lc = min(C, T - s);
    const size_t row0 = (size_t)bh * T + s;

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
    // row fragments X[16jt+tl][32m+4g+{0..3}, 32m+16+4g+{0..3}], zero past Lc
    auto load_rows = [&](const uint16_t* X, bf16x8 (&dst)[NW][NM]) {
#pragma unroll
      for (int jt = 0; jt < NW; ++jt) {
        const int j = 16 * jt + tl;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          u16x4 lo = u16x4{0, 0, 0, 0}, hi = lo;
          if (j < Lc) {
            const uint16_t* src = X + (row0 + j) * D + 32 * m + 4 * g;
            lo = *reinterpret_cast<const u16x4*>(src);
            hi = *reinterpret_cast<const u16x4*>(src + 16);
          }
          dst[jt][m] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    };
    // PREP: the chunk's processed rows of raw vectors X into prow, and the key
    // row fragments from there (zero past Lc)
    auto prep_rows = [&](const void* X, const void* hist, const float* taps) {
      PrepChunk<D, C> pc;
      pc.load(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(hist), bh, T, p.W, s, Lc, lane);
      pc.form(taps, h, p.W, p.inv_eps, prow, PS, lane);
    };
    auto load_rows_lds = [&](bf16x8 (&dst)[NW][NM]) {
#pragma unroll
      for (int jt = 0; jt < NW; ++jt) {
        const int j = 16 * jt + tl;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          u16x4 lo = u16x4{0, 0, 0, 0}, hi = lo;
          if (j < Lc) {
            const __bf16* src = prow + j * PS + 32 * m + 4 * g;
            lo = *reinterpret_cast<const u16x4*>(src);
            hi = *reinterpret_cast<const u16x4*>(src + 16);
          }
          dst[jt][m] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
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

    load_state(p.hb);
    if constexpr (PREP) {
      prep_rows(p.k, p.k_hist, p.wk);
      __syncthreads();
      load_rows_lds(kr);
    } else {
      load_rows(Kg, kr);
    }
    {
      float lg = 0.f, bt = 0.f;
      if (lane < Lc) {
        lg = logf(p.gamma[row0 + lane]);
        bt = p.beta[row0 + lane];
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(lg, o, 64);
        if (lane >= o) lg += t;
      }
      if (lane < C) {
        bcum[lane] = lg;
        betas[lane] = bt;
      }
      if constexpr (LF) {
        // Lambda[16nt+tl][32m+4g+{0..3}, 32m+16+4g+{0..3}] of the head as bf16;
        // every lane writes and later reads only its own slots
        const float* L = p.lam + (size_t)h * D * D;
#pragma unroll 4
        for (int f = 0; f < ND * NM; ++f) {
          const int nt = f / NM, m = f % NM;
          const float* src = L + (size_t)(16 * nt + tl) * D + 32 * m + 4 * g;
          lamf[f * 64 + lane] = pack8(*reinterpret_cast<const f32x4*>(src), *reinterpret_cast<const f32x4*>(src + 16));
        }
      } else {
        for (int i = lane; i < D; i += 64) lam_s[i] = p.lam[(size_t)h * D + i];
      }
    }
    __syncthreads();
    if constexpr (PREP) {
      // the key fragments are in registers: the queries replace the keys
      prep_rows(p.q, p.q_hist, p.wq);
      __syncthreads();
    }
    columns_from_rows(kr);
    pin_operands();

    // ---- per-tile machinery ----------------------------------------------------------
    float W[NW][4];   // causal decayed weights W_tj of the current tile's tokens
    float Gam = 1.f;  // Gamma_t of the current tile's token
    int w = 0;        // current tile (wave-uniform)

    // S^T <- W .* (K U^T): the causal, decayed key scores of the tile's tokens
    auto scores = [&](const bf16x8* ub, bf16x8* sb) {
      f32x4 sc[NW];
#pragma unroll
      for (int jt = 0; jt < NW; ++jt) {
        if (jt <= w) {
          sc[jt] = mfma_bf16(kr[jt][0], ub[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int m = 1; m < NM; ++m) sc[jt] = mfma_bf16(kr[jt][m], ub[m], sc[jt]);
          asm volatile("" : "+v"(sc[jt]));
        }
      }
#pragma unroll
      for (int mj = 0; mj < NMJ; ++mj) {
        if (2 * mj <= w) {
          const int jl = 2 * mj, jh = (2 * mj + 1) % NW;
          const f32x4 lo = sc[jl] * f32x4{W[jl][0], W[jl][1], W[jl][2], W[jl][3]};
          f32x4 hi = f32x4{0.f, 0.f, 0.f, 0.f};
          if (2 * mj + 1 <= w) hi = sc[jh] * f32x4{W[jh][0], W[jh][1], W[jh][2], W[jh][3]};
          sb[mj] = pack8(lo, hi);
        }
      }
    };
    // acc <- Gam * (Mb U^T) + lam .* U (when with_lambda) + Y^T S^T
    f32x4 acc[ND];
    auto product = [&](const f32x4* u, const bf16x8* ub, const bf16x8* sb, const bool with_lambda) {
#pragma unroll
      for (int nt = 0; nt < ND; ++nt) {
        f32x4 t = mfma_bf16(mf[nt][0], ub[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int m = 1; m < NM; ++m) t = mfma_bf16(mf[nt][m], ub[m], t);
        asm volatile("" : "+v"(t));
        acc[nt] = t * Gam;
        if constexpr (LF) {
          if (with_lambda) {
#pragma unroll
            for (int m = 0; m < NM; ++m) acc[nt] = mfma_bf16(lamf[(nt * NM + m) * 64 + lane], ub[m], acc[nt]);
          }
        } else {
          if (with_lambda) acc[nt] += *reinterpret_cast<const f32x4*>(&lam_s[16 * nt + 4 * g]) * u[nt];
        }
      }
#pragma unroll
      for (int mj = 0; mj < NMJ; ++mj) {
        if (2 * mj <= w) {
#pragma unroll
          for (int nt = 0; nt < ND; ++nt) acc[nt] = mfma_bf16(kc[nt][mj], sb[mj], acc[nt]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < ND; ++nt) asm volatile("" : "+v"(acc[nt]));
    };
    auto tile_constants = [&]() {
      const int tloc = 16 * w + tl;
      const bool valid = tloc < Lc;
      const float btl = bcum[tloc];
      Gam = expf(btl);
#pragma unroll
      for (int jt = 0; jt < NW; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 16 * jt + 4 * g + i;
          W[jt][i] = (jt <= w && j <= tloc && valid) ? expf(btl - bcum[j]) * betas[j] : 0.f;
        }
    };

    // ---- conjugate gradient, tile by tile -------------------------------------------
    for (int wt = 0; wt < NW; ++wt) {
      w = __builtin_amdgcn_readfirstlane(wt);
      const int tloc = 16 * w + tl;
      const bool valid = tloc < Lc;
      tile_constants();
      f32x4 r[ND], x[ND], pv[ND];
#pragma unroll
      for (int a = 0; a < ND; ++a) {
        if constexpr (PREP) {
          const u16x4 u = *reinterpret_cast<const u16x4*>(prow + tloc * PS + 16 * a + 4 * g);
          r[a] = valid ? f32x4{bf16_to_f32(u[0]), bf16_to_f32(u[1]), bf16_to_f32(u[2]), bf16_to_f32(u[3])}
                       : f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
          r[a] = valid ? load4<true>(Qg, (row0 + tloc) * D + 16 * a + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        x[a] = f32x4{0.f, 0.f, 0.f, 0.f};
        pv[a] = r[a];
      }
      if (WARM && w > 0) {
        // x_0 = token t-16's solution (the previous tile's, same lane); r_0 = q - A_t x_0
        bf16x8 ub[NM], sb[NMJ];
#pragma unroll
        for (int a = 0; a < ND; ++a) x[a] = valid ? xs[((w - 1) * ND + a) * 64 + lane] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NM; ++m) ub[m] = pack8(x[2 * m], x[2 * m + 1]);
        pin_operands();
        scores(ub, sb);
        product(x, ub, sb, true);
#pragma unroll
        for (int a = 0; a < ND; ++a) {
          r[a] -= acc[a];
          pv[a] = r[a];
        }
      }
      float rho = 0.f;
#pragma unroll
      for (int a = 0; a < ND; ++a) rho += r[a][0] * r[a][0] + r[a][1] * r[a][1] + r[a][2] * r[a][2] + r[a][3] * r[a][3];
      rho = sum_lane_groups(rho);
      int n = 0;
      bool stopped = false;
      for (int it = 0; it < p.max_steps; ++it) {
        const bool active = !stopped && rho >= kCgZero && rho > p.tol2;
        if (!__any(active)) break;
        pin_operands();
        bf16x8 ub[NM], sb[NMJ];
#pragma unroll
        for (int m = 0; m < NM; ++m) ub[m] = pack8(pv[2 * m], pv[2 * m + 1]);
        scores(ub, sb);
        product(pv, ub, sb, true);
        float pw = 0.f;
#pragma unroll
        for (int a = 0; a < ND; ++a)
          pw += pv[a][0] * acc[a][0] + pv[a][1] * acc[a][1] + pv[a][2] * acc[a][2] + pv[a][3] * acc[a][3];
        pw = sum_lane_groups(pw);
        const bool ok = active && pw >= kCgZero;
        stopped = !ok;
        const float alpha = ok ? rho * __builtin_amdgcn_rcpf(pw) : 0.f;
        float rr = 0.f;
#pragma unroll
        for (int a = 0; a < ND; ++a) {
          x[a] += alpha * pv[a];
          r[a] -= alpha * acc[a];
          rr += r[a][0] * r[a][0] + r[a][1] * r[a][1] + r[a][2] * r[a][2] + r[a][3] * r[a][3];
        }
        rr = sum_lane_groups(rr);
        // a stopped token keeps x and r (alpha = 0); its direction becomes r,
        // which stays finite and is never used again
        const float bet = ok ? rr * __builtin_amdgcn_rcpf(rho) : 0.f;
        // p <- r + bet p in place (three-operand FMA; the two-address form would
        // tie the result to r, which stays live, and cost a copy per element)
#pragma unroll
        for (int a = 0; a < ND; ++a)
#pragma unroll
          for (int i = 0; i < 4; ++i) asm("v_fma_f32 %0, %1, %0, %2" : "+v"(pv[a][i]) : "v"(bet), "v"(r[a][i]));
        rho = ok ? rr : rho;
        n += ok ? 1 : 0;
      }
#pragma unroll
      for (int a = 0; a < ND; ++a) xs[(w * ND + a) * 64 + lane] = x[a];
      if (valid) {
        if (p.x_out) {
#pragma unroll
          for (int a = 0; a < ND; ++a)
            *reinterpret_cast<f32x4*>(p.x_out + (row0 + tloc) * D + 16 * a + 4 * g) = x[a];
        }
        if (p.steps && g == 0) p.steps[row0 + tloc] = n;
      }
    }

    // ---- read-out o_t = Gamma_t Gb x_t + sum_j W_tj (k_j . x_t) v_j ------------------
    // Gb and the value columns replace Hb and the key columns (the key rows stay:
    // the scores of x are against the keys).  No read-out without o (solutions only).
    if (p.o) {
    load_state(p.gb);
    {
      bf16x8 vr[NW][NM];
      load_rows(Vg, vr);
      columns_from_rows(vr);
    }
    pin_operands();
    for (int wt = 0; wt < NW; ++wt) {
      w = __builtin_amdgcn_readfirstlane(wt);
      const int tloc = 16 * w + tl;
      tile_constants();
      f32x4 x[ND];
#pragma unroll
      for (int a = 0; a < ND; ++a) x[a] = xs[(w * ND + a) * 64 + lane];
      bf16x8 xb[NM], sb[NMJ];
#pragma unroll
      for (int m = 0; m < NM; ++m) xb[m] = pack8(x[2 * m], x[2 * m + 1]);
      scores(xb, sb);
      pin_operands();
      product(x, xb, sb, false);
      if (tloc < Lc) {
#pragma unroll
        for (int a = 0; a < ND; ++a)
          *reinterpret_cast<f32x4*>(p.o + (row0 + tloc) * D + 16 * a + 4 * g) = acc[a];
      }
    }
    }
    __syncthreads();  // the next chunk rewrites the gates and Lambda in LDS
  }
}

template <int D, int C, bool LF = false>
hipError_t launch_t(const CgParams& p, hipStream_t s) {
  const long long chunks = (long long)p.BH * p.NC;
  const dim3 grid((unsigned)((chunks + kChunksPerWave - 1) / kChunksPerWave));
  if constexpr (!LF) {
    if (p.prep) {
      if constexpr (C == 64 && D >= 64) {
        if (p.warm) return hipErrorInvalidValue;
        hipLaunchKernelGGL((cg_bf16_unscaled_kernel<D, C, false, false, true>), grid, dim3(64), 0, s, p);
      } else {
        return hipErrorInvalidValue;
      }
    } else if (p.warm) {
      hipLaunchKernelGGL((cg_bf16_unscaled_kernel<D, C, false, true>), grid, dim3(64), 0, s, p);
    } else {
      hipLaunchKernelGGL((cg_bf16_unscaled_kernel<D, C, false, false>), grid, dim3(64), 0, s, p);
    }
  } else {
    if (p.warm || p.prep) return hipErrorInvalidValue;
    hipLaunchKernelGGL((cg_bf16_unscaled_kernel<D, C, LF>), grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
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

hipError_t launch_cg_bf16_unscaled(int D, int C, const CgParams& p, hipStream_t s) {
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
