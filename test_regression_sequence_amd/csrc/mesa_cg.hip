// Chunked conjugate-gradient solve and read-out of the Mesa layer, fp32
// inputs (fp32 MFMA).  bf16 inputs take the tuned kernels of mesa_cg_bf16.hip.
//
// MesaNet page, technical summary, "Mesa layer" section: the optimal query
// response x_t = (H_t + Lambda)^{-1} q_t is found by conjugate gradient, the
// output is o_t = G_t x_t, the step count per token follows a stopping
// criterion ("dynamic compute"), and the work is parallel over chunks
// (parallelisation paragraph).  Inside chunk c (tokens s..s+C-1, boundary
// states Hb = H_{s-1}, Gb = G_{s-1}):
//
//   b_t = sum_{i=s..t} log gamma_i,  Gamma_t = e^{b_t},
//   W_tj = e^{b_t - b_j} beta_j for j <= t (else 0),
//   H_t p = Gamma_t Hb p + sum_{j<=t} W_tj (k_j . p) k_j,
//   o_t   = Gamma_t Gb x_t + sum_{j<=t} W_tj (k_j . x_t) v_j.
//
// One workgroup per chunk, one wave per 16 tokens; the waves never
// synchronise inside the CG loop (every token's iteration touches only its
// own vectors and read-only chunk data), so each wave leaves the loop as soon
// as its 16 tokens have stopped.  All matrix products run on 16x16x4 fp32
// MFMA in a transposed orientation: the per-token vectors are the B operand,
// so lane l of a wave holds token 16w + l%16 and dims 16a + 4(l/16) + {0..3}
// of every CG vector, MFMA results land directly in that layout, and the CG
// scalars need only a 4-lane reduction.  The boundary state and the chunk's
// keys and values sit in LDS.
#include "mesa_common.h"
#include "mesa_kernels.h"

namespace mesa {

namespace {

template <int D, int C>
struct CgLds {
  static constexpr int S = D + 1;
  float M[D * S];                      // Hb during CG, Gb for the read-out, [row][col]
  float Ks[C * S];                     // K chunk [token][dim]
  float Vs[C * S];                     // V chunk [token][dim]
};

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

template <int D, int C>
__global__ __launch_bounds__(64 * (C / 16)) void cg_kernel(CgParams p) {
  constexpr int ND = D / 16;   // dim tiles
  constexpr int NW = C / 16;   // waves = token tiles
  using L = CgLds<D, C>;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, tl = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / p.NC, c = blockIdx.x % p.NC;
  const int h = bh % p.H;
  const int T = p.T, s = c * C, Lc = min(C, T - s);
  const size_t row0 = (size_t)bh * T + s;
  const int tloc = 16 * w + tl;
  const bool valid = tloc < Lc;

  __shared__ float bcum[C];
  __shared__ float betas[C];
  __shared__ __attribute__((aligned(16))) L lds;

  // ---- gate prefix b_t (wave 0, inclusive scan) ------------------------------
  if (w == 0) {
    float v = 0.f, bt = 0.f;
    if (lane < C && lane < Lc) {
      v = logf(p.gamma[row0 + lane]);
      bt = p.beta[row0 + lane];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_up(v, o, 64);
      if (lane >= o) v += t;
    }
    if (lane < C) {
      bcum[lane] = v;
      betas[lane] = bt;
    }
  }

  // ---- stage the chunk's keys, values and boundary state ----------------------
  {
    constexpr int S = L::S;
    const float* Kg = static_cast<const float*>(p.k);
    const float* Vg = static_cast<const float*>(p.v);
    const float* Hg = static_cast<const float*>(p.hb) + ((size_t)bh * p.NC + c) * D * D;
    for (int pc = tid; pc < C * D; pc += 64 * NW) {
      const int j = pc / D, d = pc % D;
      lds.Ks[j * S + d] = (j < Lc) ? Kg[(row0 + j) * D + d] : 0.f;
      lds.Vs[j * S + d] = (j < Lc) ? Vg[(row0 + j) * D + d] : 0.f;
    }
    for (int pc = tid; pc < D * D; pc += 64 * NW) lds.M[(pc / D) * S + pc % D] = Hg[pc];
  }
  __syncthreads();

  // ---- per-token constants ----------------------------------------------------
  const float bt = bcum[tloc];
  const float Gam = __expf(bt);
  float W[NW][4];
#pragma unroll
  for (int jt = 0; jt < NW; ++jt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * jt + 4 * g + i;
      W[jt][i] = (jt <= w && j <= tloc && valid) ? __expf(bt - bcum[j]) * betas[j] : 0.f;
    }
  f32x4 lam[ND], r[ND], x[ND], pv[ND], acc[ND];
#pragma unroll
  for (int a = 0; a < ND; ++a) {
    lam[a] = *reinterpret_cast<const f32x4*>(p.lam + (size_t)h * D + 16 * a + 4 * g);
    r[a] = valid ? load4<false>(p.q, (row0 + tloc) * D + 16 * a + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
    x[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    pv[a] = r[a];
  }

  // y <- A y-operand: Gamma_t * Mb u + (sum_j W_tj (k_j.u) Y_j) for u = src
  // (Mb = Hb or Gb, Y = K or V); returns through out[].
  auto chunk_product = [&](const f32x4* src, f32x4* out, bool use_values) {
    f32x4 sc[NW];
    constexpr int S = L::S;
#pragma unroll
    for (int nt = 0; nt < ND; ++nt) {
      f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int a = 0; a < ND; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) t = mfma_f32(lds.M[(16 * nt + tl) * S + 16 * a + 4 * g + i], src[a][i], t);
      out[nt] = t * Gam;
    }
#pragma unroll
    for (int jt = 0; jt < NW; ++jt) {
      if (jt > w) continue;
      f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int a = 0; a < ND; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) t = mfma_f32(lds.Ks[(16 * jt + tl) * S + 16 * a + 4 * g + i], src[a][i], t);
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] *= W[jt][i];
      sc[jt] = t;
    }
    const float* Y = use_values ? lds.Vs : lds.Ks;
#pragma unroll
    for (int nt = 0; nt < ND; ++nt)
#pragma unroll
      for (int jt = 0; jt < NW; ++jt) {
        if (jt > w) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[nt] = mfma_f32(Y[(16 * jt + 4 * g + i) * S + 16 * nt + tl], sc[jt][i], out[nt]);
      }
  };

  // ---- conjugate gradient -----------------------------------------------------
  float rho = 0.f;
#pragma unroll
  for (int a = 0; a < ND; ++a) rho += dot4(r[a], r[a]);
  rho = sum_lane_groups(rho);
  int n = 0;
  bool stopped = false;
  for (int it = 0; it < p.max_steps; ++it) {
    const bool active = !stopped && rho >= kCgZero && rho > p.tol2;
    if (!__any(active)) break;
    chunk_product(pv, acc, false);
    float pw = 0.f;
#pragma unroll
    for (int a = 0; a < ND; ++a) {
      acc[a] += lam[a] * pv[a];
      pw += dot4(pv[a], acc[a]);
    }
    pw = sum_lane_groups(pw);
    const bool ok = active && pw >= kCgZero;
    stopped = !ok;
    const float alpha = ok ? rho / pw : 0.f;
    float rr = 0.f;
#pragma unroll
    for (int a = 0; a < ND; ++a) {
      x[a] += alpha * pv[a];
      r[a] -= alpha * acc[a];
      rr += dot4(r[a], r[a]);
    }
    rr = sum_lane_groups(rr);
    const float bet = ok ? rr / rho : 0.f;
#pragma unroll
    for (int a = 0; a < ND; ++a) pv[a] = ok ? r[a] + bet * pv[a] : pv[a];
    rho = ok ? rr : rho;
    n += ok ? 1 : 0;
  }

  // ---- read-out o_t = G_t x_t -------------------------------------------------
  {
    constexpr int S = L::S;
    __syncthreads();  // every wave is done reading Hb
    const float* Gg = static_cast<const float*>(p.gb) + ((size_t)bh * p.NC + c) * D * D;
    for (int pc = tid; pc < D * D; pc += 64 * NW) lds.M[(pc / D) * S + pc % D] = Gg[pc];
    __syncthreads();
  }
  chunk_product(x, acc, true);

  if (valid) {
    const size_t orow = (row0 + tloc) * D;
#pragma unroll
    for (int a = 0; a < ND; ++a) *reinterpret_cast<f32x4*>(p.o + orow + 16 * a + 4 * g) = acc[a];
    if (p.x_out) {
#pragma unroll
      for (int a = 0; a < ND; ++a) *reinterpret_cast<f32x4*>(p.x_out + orow + 16 * a + 4 * g) = x[a];
    }
    if (p.steps && g == 0) p.steps[row0 + tloc] = n;
  }
}

template <int D, int C>
hipError_t launch_cg_t(const CgParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.BH * p.NC);
  hipLaunchKernelGGL((cg_kernel<D, C>), grid, dim3(64 * (C / 16)), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_cg_d(int C, const CgParams& p, hipStream_t s) {
  switch (C) {
    case 16: return launch_cg_t<D, 16>(p, s);
    case 32: return launch_cg_t<D, 32>(p, s);
    case 64: return launch_cg_t<D, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_cg(bool bf16, int D, int C, const CgParams& p, hipStream_t s) {
  if (bf16) return launch_cg_bf16(D, C, p, s);
  switch (D) {
    case 16: return launch_cg_d<16>(C, p, s);
    case 32: return launch_cg_d<32>(C, p, s);
    case 64: return launch_cg_d<64>(C, p, s);
    case 128: return launch_cg_d<128>(C, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mesa
