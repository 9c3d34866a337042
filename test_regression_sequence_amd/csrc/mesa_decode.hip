// Recurrent decode step of the Mesa layer (one new token per sequence).
//
// MesaNet page, technical summary, "Mesa layer" section: the recurrent form
// costs O(1) per token -- update the two states with the new token,
//     H <- gamma H + beta k k^T,   G <- gamma G + beta v k^T,
// solve (H + Lambda) x = q by conjugate gradient (fixed steps or residual
// test), emit o = G x.  The step is bound by streaming H and G through HBM
// (2 * 4 * d^2 bytes read and written per (sequence, head) pair); the CG
// iterations run on the register-resident H between the two streams.
//
// One workgroup of 256 threads per pair.  Thread (rg, j) owns column j of H
// for the rows of row group rg; a row of H is read and written by D
// consecutive threads, so the H stream is fully coalesced.  H is symmetric,
// so column j equals row j and the matrix-vector product needs only a
// broadcast of p (LDS) and a sum over the row groups.  The update forms
// k_r*k_j before scaling, so an exactly symmetric H stays exactly symmetric.
#include "mesa_common.h"
#include "mesa_kernels.h"

namespace mesa {

namespace {

constexpr int kDecThreads = 256;

template <int NWAVES>
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) s += red[i];
  __syncthreads();
  return s;
}

template <bool BF16, int D>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeParams p) {
  constexpr int RG = kDecThreads / D;  // row groups
  constexpr int RPT = D / RG;          // rows of H per thread
  constexpr int NWV = kDecThreads / 64;
  const int pair = blockIdx.x;
  const int h = pair % p.H;
  const int tid = threadIdx.x, j = tid % D, rg = tid / D;

  __shared__ float ks[D], qs[D], vs[D], xs[D], pvec[D];
  __shared__ float part[RG][D];
  __shared__ float red[NWV];

  if (tid < D) {
    ks[tid] = load1<BF16>(p.k, (size_t)pair * D + tid);
    qs[tid] = load1<BF16>(p.q, (size_t)pair * D + tid);
    vs[tid] = load1<BF16>(p.v, (size_t)pair * D + tid);
  }
  const float gam = p.gamma[pair], bet = p.beta[pair];
  __syncthreads();

  // ---- H <- gamma H + beta (k k^T), kept in registers --------------------------
  float* Hp = p.h + (size_t)pair * D * D;
  float hreg[RPT];
  const float kj = ks[j];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg * RPT + i;
    hreg[i] = Hp[(size_t)row * D + j];
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg * RPT + i;
    const float hv = gam * hreg[i] + bet * (ks[row] * kj);
    hreg[i] = hv;
    Hp[(size_t)row * D + j] = hv;
  }

  // ---- CG on (H + Lambda) x = q; vector index j lives in thread j (rg == 0) ----
  const bool owner = rg == 0;
  const float lamj = p.lam[(size_t)h * D + j];
  float xj = 0.f, rj = owner ? qs[j] : 0.f, pj = rj;
  float rho = block_sum<NWV>(rj * rj, red);
  int n = 0;
  for (int it = 0; it < p.max_steps; ++it) {
    if (!(rho > 0.f && rho > p.tol2)) break;
    if (owner) pvec[j] = pj;
    __syncthreads();
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) acc += hreg[i] * pvec[rg * RPT + i];
    part[rg][j] = acc;
    __syncthreads();
    float wj = 0.f;
    if (owner) {
#pragma unroll
      for (int q = 0; q < RG; ++q) wj += part[q][j];
      wj += lamj * pj;
    }
    const float pw = block_sum<NWV>(pj * wj, red);
    if (!(pw > 0.f)) break;
    const float alpha = rho / pw;
    xj += alpha * pj;
    rj -= alpha * wj;
    const float rr = block_sum<NWV>(rj * rj, red);
    pj = rj + (rr / rho) * pj;
    rho = rr;
    ++n;
  }
  if (owner) xs[j] = xj;
  __syncthreads();

  // ---- G <- gamma G + beta (v k^T); o = G x ------------------------------------
  float* Gp = p.g + (size_t)pair * D * D;
  if (tid < D) {
    const int row = tid;
    const float bv = bet * vs[row];
    float o = 0.f;
#pragma unroll 4
    for (int c4 = 0; c4 < D / 4; ++c4) {
      f32x4 gv = *reinterpret_cast<const f32x4*>(Gp + (size_t)row * D + 4 * c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gv[e] = gam * gv[e] + bv * ks[4 * c4 + e];
        o += gv[e] * xs[4 * c4 + e];
      }
      *reinterpret_cast<f32x4*>(Gp + (size_t)row * D + 4 * c4) = gv;
    }
    p.o[(size_t)pair * D + row] = o;
    if (p.x_out) p.x_out[(size_t)pair * D + row] = xs[row];
  }
  if (tid == 0 && p.steps) p.steps[pair] = n;
}

template <bool BF16, int D>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<BF16, D>), dim3(p.P), dim3(kDecThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(bool bf16, int D, const DecodeParams& p, hipStream_t s) {
  if (bf16) {
    if (D == 128) return launch_decode_t<true, 128>(p, s);
    if (D == 64) return launch_decode_t<true, 64>(p, s);
  } else {
    if (D == 128) return launch_decode_t<false, 128>(p, s);
    if (D == 64) return launch_decode_t<false, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mesa
