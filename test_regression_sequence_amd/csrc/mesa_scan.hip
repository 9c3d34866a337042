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
// Work split: one workgroup (4 waves) per (b, h, state in {H, G}, 16-row
// stripe of the state), so a (b, h) uses 2*D/16 workgroups that the launch
// maps onto one XCD (they share the chunk's keys through that XCD's L2).
// The chunk delta K^T diag(w) X is an MFMA contraction over the chunk's
// tokens: bf16 MFMA for bf16 inputs with the scaled operand split into
// bf16 hi + lo parts (so the carried fp32 state does not pick up a bf16
// rounding of beta*tail*x), fp32 MFMA for fp32 inputs.
//
// Snapshot layouts (consumed only by the CG kernel):
//   fp32 path: row-major [D][D] fp32, H[r][c] and G[v][k].
//   bf16 path: MFMA A-operand fragments.  Fragment f = nt*(D/32) + m holds,
//     for lane l (tl = l%16, g = l/16), 8 bf16: row 16*nt + tl, columns
//     32m + 4g + {0..3} then 32m + 16 + 4g + {0..3}.  Stored [f][lane][8].
#include "mesa_common.h"
#include "mesa_kernels.h"

namespace mesa {

namespace {

constexpr int kScanThreads = 256;

template <bool BF16, int D, int C>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(ScanParams p) {
  constexpr int ND = D / 16;          // 16-wide tiles per state dimension
  constexpr int TPW = (ND + 3) / 4;   // state tiles owned by each wave
  constexpr int CP = (C < 32) ? 32 : C;  // token dim padded to one bf16 MFMA k-block
  constexpr int U = 2 * ND;           // workgroups per (b, h)

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, tl = lane & 15, g = lane >> 4;

  // XCD-aware decode: the U workgroups of one (b, h) share blockIdx % 8.
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  const int bh = (local / U) * 8 + xcd;
  if (bh >= p.BH) return;
  const int u = local % U;
  const int which = u / ND;           // 0: H, 1: G
  const int mt = u % ND;              // 16-row stripe of the (H or G^T) state

  const int T = p.T, NC = p.NC;
  const void* X = which ? p.v : p.k;  // the second factor of the chunk delta
  const size_t row0 = (size_t)bh * T;

  __shared__ float logg[C];
  __shared__ float wsc[C];            // beta_j * tail_j
  __shared__ float gamma_c;
  // A operand: K restricted to this stripe's 16 state rows; B operand: w .* X.
  __shared__ __attribute__((aligned(16))) char lds_a[BF16 ? 16 * (CP + 8) * 2 : CP * 16 * 4];
  __shared__ __attribute__((aligned(16))) char lds_b[BF16 ? 2 * D * (CP + 8) * 2 : CP * D * 4];

  // Running state.  Tile ti of this wave is (mt, nt = wave + 4 ti); lane holds
  // O[16 mt + 4 g + i][16 nt + tl], where O = H for H and O = G^T for G.
  f32x4 st[TPW];
  const float* init = which ? p.g0 : p.h0;
#pragma unroll
  for (int ti = 0; ti < TPW; ++ti) {
    const int nt = wave + 4 * ti;
    st[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nt < ND && init) {
      const float* base = init + (size_t)bh * D * D;
      if (which == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st[ti][i] = base[(size_t)(16 * mt + 4 * g + i) * D + 16 * nt + tl];
      } else {
        st[ti] = *reinterpret_cast<const f32x4*>(base + (size_t)(16 * nt + tl) * D + 16 * mt + 4 * g);
      }
    }
  }

  for (int c = 0; c < NC; ++c) {
    const int s = c * C;
    const int Lc = min(C, T - s);

    // ---- snapshot of the state before chunk c --------------------------------
    {
      const size_t snap = ((size_t)bh * NC + c) * D * D;
#pragma unroll
      for (int ti = 0; ti < TPW; ++ti) {
        const int nt = wave + 4 * ti;
        if (nt >= ND) continue;
        if constexpr (BF16) {
          __bf16* dst = static_cast<__bf16*>(which ? p.gb : p.hb) + snap;
          const int frag = nt * (ND / 2) + (mt >> 1);
          bf16x4 h4;
#pragma unroll
          for (int i = 0; i < 4; ++i) h4[i] = (__bf16)st[ti][i];
          *reinterpret_cast<bf16x4*>(dst + ((size_t)frag * 64 + lane) * 8 + 4 * (mt & 1)) = h4;
        } else {
          float* dst = static_cast<float*>(which ? p.gb : p.hb) + snap;
          if (which == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(size_t)(16 * mt + 4 * g + i) * D + 16 * nt + tl] = st[ti][i];
          } else {
            *reinterpret_cast<f32x4*>(dst + (size_t)(16 * nt + tl) * D + 16 * mt + 4 * g) = st[ti];
          }
        }
      }
    }

    // ---- gates: w_j = beta_j * prod_{i=j+1..e} gamma_i, Gamma_c --------------
    __syncthreads();  // previous chunk's readers of the LDS buffers are done
    if (tid < C) logg[tid] = (tid < Lc) ? logf(p.gamma[row0 + s + tid]) : 0.f;
    __syncthreads();
    if (tid < C) {
      float suf = 0.f;
      for (int i = tid + 1; i < Lc; ++i) suf += logg[i];
      wsc[tid] = (tid < Lc) ? p.beta[row0 + s + tid] * expf(suf) : 0.f;
      if (tid == 0) gamma_c = (Lc > 0) ? expf(suf + logg[0]) : 1.f;
    }
    __syncthreads();

    // ---- stage operands ------------------------------------------------------
    if constexpr (BF16) {
      __bf16* KT = reinterpret_cast<__bf16*>(lds_a);              // [16][CP+8]
      __bf16* XH = reinterpret_cast<__bf16*>(lds_b);              // [D][CP+8]
      __bf16* XL = XH + D * (CP + 8);                             // [D][CP+8]
      const uint16_t* Xg = static_cast<const uint16_t*>(X);
      const uint16_t* Kg = static_cast<const uint16_t*>(p.k);
      // pieces: (token pair jp, 8-column group c8); one dword LDS write per column
      constexpr int NP = (CP / 2) * (D / 8);
      for (int pc = tid; pc < NP; pc += kScanThreads) {
        const int jp = pc % (CP / 2), c8 = pc / (CP / 2);
        const int j0 = 2 * jp, j1 = j0 + 1;
        u16x8 a = u16x8{0, 0, 0, 0, 0, 0, 0, 0}, b = a;
        if (j0 < Lc) a = *reinterpret_cast<const u16x8*>(Xg + (row0 + s + j0) * D + 8 * c8);
        if (j1 < Lc) b = *reinterpret_cast<const u16x8*>(Xg + (row0 + s + j1) * D + 8 * c8);
        const float w0 = (j0 < Lc) ? wsc[j0] : 0.f, w1 = (j1 < Lc) ? wsc[j1] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x0 = w0 * bf16_to_f32(a[e]), x1 = w1 * bf16_to_f32(b[e]);
          const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
          const __bf16 l0 = (__bf16)(x0 - (float)h0), l1 = (__bf16)(x1 - (float)h1);
          const int n = 8 * c8 + e;
          *reinterpret_cast<uint32_t*>(XH + n * (CP + 8) + j0) = pack2(h0, h1);
          *reinterpret_cast<uint32_t*>(XL + n * (CP + 8) + j0) = pack2(l0, l1);
        }
      }
      // A operand: K^T rows 16 mt .. 16 mt + 15
      for (int pc = tid; pc < (CP / 2) * 2; pc += kScanThreads) {
        const int jp = pc % (CP / 2), half = pc / (CP / 2);
        const int j0 = 2 * jp, j1 = j0 + 1;
        u16x8 a = u16x8{0, 0, 0, 0, 0, 0, 0, 0}, b = a;
        if (j0 < Lc) a = *reinterpret_cast<const u16x8*>(Kg + (row0 + s + j0) * D + 16 * mt + 8 * half);
        if (j1 < Lc) b = *reinterpret_cast<const u16x8*>(Kg + (row0 + s + j1) * D + 16 * mt + 8 * half);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = 8 * half + e;
          *reinterpret_cast<uint32_t*>(KT + m * (CP + 8) + j0) =
              (uint32_t)a[e] | ((uint32_t)b[e] << 16);
        }
      }
    } else {
      float* Ks = reinterpret_cast<float*>(lds_a);                // [CP][16]
      float* Xs = reinterpret_cast<float*>(lds_b);                // [CP][D] = w_j * X[j][n]
      const float* Xg = static_cast<const float*>(X);
      const float* Kg = static_cast<const float*>(p.k);
      for (int pc = tid; pc < C * (D / 4); pc += kScanThreads) {
        const int j = pc / (D / 4), c4 = pc % (D / 4);
        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j < Lc) a = *reinterpret_cast<const f32x4*>(Xg + (row0 + s + j) * D + 4 * c4) * wsc[j];
        *reinterpret_cast<f32x4*>(Xs + j * D + 4 * c4) = a;
      }
      for (int pc = tid; pc < C * 4; pc += kScanThreads) {
        const int j = pc / 4, c4 = pc % 4;
        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
        if (j < Lc) a = *reinterpret_cast<const f32x4*>(Kg + (row0 + s + j) * D + 16 * mt + 4 * c4);
        *reinterpret_cast<f32x4*>(Ks + j * 16 + 4 * c4) = a;
      }
    }
    __syncthreads();

    // ---- delta tiles and state update ----------------------------------------
    const float gc = gamma_c;
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      const int nt = wave + 4 * ti;
      if (nt >= ND) continue;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
        const __bf16* KT = reinterpret_cast<const __bf16*>(lds_a);
        const __bf16* XH = reinterpret_cast<const __bf16*>(lds_b);
        const __bf16* XL = XH + D * (CP + 8);
#pragma unroll
        for (int kb = 0; kb < CP / 32; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(KT + tl * (CP + 8) + 32 * kb + 8 * g);
          const bf16x8 bh_ = *reinterpret_cast<const bf16x8*>(XH + (16 * nt + tl) * (CP + 8) + 32 * kb + 8 * g);
          const bf16x8 bl_ = *reinterpret_cast<const bf16x8*>(XL + (16 * nt + tl) * (CP + 8) + 32 * kb + 8 * g);
          acc = mfma_bf16(a, bh_, acc);
          acc = mfma_bf16(a, bl_, acc);
        }
      } else {
        const float* Ks = reinterpret_cast<const float*>(lds_a);
        const float* Xs = reinterpret_cast<const float*>(lds_b);
#pragma unroll 4
        for (int kb = 0; kb < C / 4; ++kb) {
          acc = mfma_f32(Ks[(4 * kb + g) * 16 + tl], Xs[(4 * kb + g) * D + 16 * nt + tl], acc);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) st[ti][i] = gc * st[ti][i] + acc[i];
    }
  }

  // ---- final state (fp32, row-major) ------------------------------------------
  float* fin = which ? p.g_final : p.h_final;
  if (fin) {
    float* base = fin + (size_t)bh * D * D;
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      const int nt = wave + 4 * ti;
      if (nt >= ND) continue;
      if (which == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) base[(size_t)(16 * mt + 4 * g + i) * D + 16 * nt + tl] = st[ti][i];
      } else {
        *reinterpret_cast<f32x4*>(base + (size_t)(16 * nt + tl) * D + 16 * mt + 4 * g) = st[ti];
      }
    }
  }
}

template <bool BF16, int D, int C>
hipError_t launch_scan_t(const ScanParams& p, hipStream_t s) {
  constexpr int U = 2 * (D / 16);
  const int groups = (p.BH + 7) / 8;
  const dim3 grid(groups * 8 * U);
  hipLaunchKernelGGL((scan_kernel<BF16, D, C>), grid, dim3(kScanThreads), 0, s, p);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_scan_d(int C, const ScanParams& p, hipStream_t s) {
  switch (C) {
    case 16: return launch_scan_t<BF16, D, 16>(p, s);
    case 32: return launch_scan_t<BF16, D, 32>(p, s);
    case 64: return launch_scan_t<BF16, D, 64>(p, s);
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
