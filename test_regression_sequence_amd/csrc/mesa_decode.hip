// Recurrent decode step of the Mesa layer (one new token per sequence).
//
// MesaNet page, technical summary, "Mesa layer" section: the recurrent form
// costs O(1) per token -- update the two states with the new token,
//     H <- gamma H + beta k k^T,   G <- gamma G + beta v k^T,
// solve (H + Lambda) x = q by conjugate gradient (fixed steps or residual
// test), emit o = G x.  The step is bound by streaming H and G through HBM
// (2 * 4 * d^2 bytes read and written per (sequence, head) pair); the CG
// iterations run on the register-resident H while G's loads are in flight,
// and two pairs share each CU, so one pair's solve overlaps the other's
// streams.
//
// One workgroup of NW = 4 waves per pair; both states move as 16-byte row
// segments, every wave instruction covering 1 KB of contiguous memory.
//   H: thread t holds the 4 columns 4(t % Q) .. +3 (Q = D/4 column quads) of
//      R consecutive rows (R = D*Q/(64 NW)).  H is symmetric, so y = H p is
//      the column sums sum_r H[r][j] p_r: a thread forms its part for 4
//      columns, the row groups of a wave combine by lane swaps, and the waves
//      combine through LDS at the iteration's single barrier.
//   CG vectors: every wave keeps all D entries (lane l holds entries l + 64e),
//      so both dot products are wave-local and all waves take identical
//      decisions.
//   G: the same row segments; o = G x is reduced across the lanes of a row.
// WARM: CG starts from a given x_0 (the previous token's solution, kept per
// pair by the caller) with r_0 = q - (H + Lambda) x_0, one more product with
// H + Lambda that is not counted as a step; the solution is written back in
// place of x_0.
// A full symmetric positive definite Lambda (DecodeParams::lam_full, [H, D, D])
// is added to the register copy of H after H is written back, so the CG runs
// on H + Lambda directly; the per-head Lambda is shared by all sequences of a
// head and read through the cache, each thread's strip of it loaded together
// with the state.
// The update forms k_r*k_j before scaling and is one explicit FMA per element,
// gamma*h + (beta*(k_r*k_j)), so an exactly symmetric H stays exactly
// symmetric and every variant of the kernel rounds the same way.
#include "mesa_common.h"
#include "mesa_kernels.h"

namespace mesa {

namespace {

constexpr int kDecWaves = 4;

// row-major index of block (bi, bj), bi <= bj, in the upper triangle of an nb x nb grid
__device__ __forceinline__ int sym_block(int nb, int bi, int bj) { return bi * nb - bi * (bi - 1) / 2 + (bj - bi); }

// SYMH: H is stored packed as 16x16 blocks on and above the block diagonal
// (row-major block order, each block row-major).  The workgroup streams the
// stored blocks once, contiguously, into LDS; every thread then takes its
// strip from there: on or above the diagonal straight out of its block, below
// it transposed out of the mirror block (16-byte runs of that block's rows,
// every 4x4 group transposed in registers).  The LDS copy swizzles 16-byte
// slots so that both read patterns and the linear fill avoid bank conflicts,
// and the CG buffers reuse its space.  Only threads of stored blocks write H
// back.  The CG and G parts are unchanged.
template <bool BF16, int D, bool SYMH, bool WARM>
__global__ __launch_bounds__(64 * kDecWaves) void decode_kernel(DecodeParams p) {
  constexpr int NW = kDecWaves;
  constexpr int Q = D / 4;                   // 16-byte column quads per row
  constexpr int TPR = 64 / Q;                // row groups per wave (lanes sharing a quad)
  constexpr int RPT = D / (NW * TPR);        // rows per thread
  constexpr int EPL = D / 64;                // CG vector entries per lane
  static_assert(TPR == 2 || TPR == 4, "a wave holds 2 or 4 row groups");
  static_assert(RPT % 4 == 0, "rows per thread in fours");
  const int pair = blockIdx.x;
  const int h = pair % p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int cq = lane % Q;                       // column quad
  const int row0 = (wave * TPR + lane / Q) * RPT;  // first row of this thread

  constexpr int NB = D / 16, NBLK = NB * (NB + 1) / 2;  // packed H: blocks per side, stored blocks
  constexpr int CG_LDS = 3 * NW * D;                       // floats of pb and part
  constexpr int LDS_F = SYMH && NBLK * 256 > CG_LDS ? NBLK * 256 : CG_LDS;
  __shared__ float ks[D], qs[D], vs[D], lam_s[D];
  __shared__ __attribute__((aligned(16))) float lds[LDS_F];  // packed H staging (SYMH), then pb and part
  float(*pb)[D] = reinterpret_cast<float(*)[D]>(lds);             // per-wave copy of p, then x
  float(*part2)[NW][D] = reinterpret_cast<float(*)[NW][D]>(lds + NW * D);  // per-wave column sums, double buffered

  // token vectors: one element per thread (index clamped, so the loads are
  // unconditional and the state loads below go out without waiting on them)
  static_assert(D <= 64 * NW, "one vector element per thread");
  const int iv = min(tid, D - 1);
  const float kv = load1<BF16>(p.k, (size_t)pair * D + iv);
  const float qv = load1<BF16>(p.q, (size_t)pair * D + iv);
  const float vv = load1<BF16>(p.v, (size_t)pair * D + iv);
  const float lamv = p.lam[(size_t)h * D + iv];
  const float gam = p.gamma[pair], bet = p.beta[pair];
  float x0v[WARM ? EPL : 1];  // warm start, in flight while H streams
  if constexpr (WARM) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) x0v[e] = p.x0[(size_t)pair * D + lane + 64 * e];
  }

  // ---- H <- gamma H + beta (k k^T), kept in registers, written back --------------
  // wave-uniform base plus a 32-bit per-lane byte offset (row0, cq) plus a
  // constant per row: lets every row share one address register.  The states
  // are touched once per step, so they stream with nontemporal hints (each
  // wave then covers its 16 KB of a state contiguously at full HBM rate).
  char* Gb = reinterpret_cast<char*>(p.g + (size_t)pair * D * D);
  const uint64_t voff = (uint32_t)((row0 * D + 4 * cq) * 4);
  auto at = [&](char* base, int i) { return reinterpret_cast<f32x4*>(base + voff + i * D * 4); };
  f32x4 hreg[RPT];
  // full layout
  char* Hb = reinterpret_cast<char*>(p.h + (size_t)pair * D * D);
  // packed layout
  const int bi = row0 >> 4, bj = cq >> 2, r0 = row0 & 15, cm = cq & 3;
  const bool mirror = SYMH && bi > bj;
  const int myblk = mirror ? sym_block(NB, bj, bi) : sym_block(NB, bi, bj);
  f32x4* Hp = reinterpret_cast<f32x4*>(p.h + (size_t)pair * NBLK * 256);
  // 16-byte slot of (row, column quad c4) of stored block blk in the LDS copy
  auto slot = [](int blk, int row, int c4) {
    return blk * 64 + (row >> 2) * 16 + (((row & 3) ^ (blk & 3)) << 2) + (c4 ^ ((row >> 2) & 3));
  };
  // this thread's j-th row segment: direct, or the transposed source in the mirror block
  auto strip = [&](int j) {
    return mirror ? slot(myblk, 4 * cm + (j & 3), (r0 >> 2) + (j >> 2)) : slot(myblk, r0 + j, cm);
  };
  auto transpose_groups = [&]() {  // mirror threads: out[4g+u][e] = in[4g+e][u]
#pragma unroll
    for (int g4 = 0; g4 < RPT / 4; ++g4) {
      f32x4 t[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) t[u][e] = mirror ? hreg[4 * g4 + e][u] : hreg[4 * g4 + u][e];
#pragma unroll
      for (int u = 0; u < 4; ++u) hreg[4 * g4 + u] = t[u];
    }
  };
  constexpr int NV = (NBLK * 64 + 64 * NW - 1) / (64 * NW);  // packed H: 16-byte loads per thread
  f32x4 stage[SYMH ? NV : 1];
  if constexpr (SYMH) {
#pragma unroll
    for (int i = 0; i < NV; ++i) stage[i] = Hp[min(tid + 64 * NW * i, NBLK * 64 - 1)];
  } else {
#pragma unroll
    for (int i = 0; i < RPT; ++i) hreg[i] = __builtin_nontemporal_load(at(Hb, i));
  }
  // a full Lambda: this thread's strip of it, in flight with the state
  const bool lam_full = p.lam_full != 0;
  f32x4 lreg[RPT];
  if (lam_full) {
    const char* Lb = reinterpret_cast<const char*>(p.lam + (size_t)h * D * D);
#pragma unroll
    for (int i = 0; i < RPT; ++i) lreg[i] = *reinterpret_cast<const f32x4*>(Lb + voff + i * D * 4);
  }
  if (tid < D) {
    ks[tid] = kv;
    qs[tid] = qv;
    vs[tid] = vv;
    lam_s[tid] = lamv;
  }
  if constexpr (SYMH) {
    f32x4* hl = reinterpret_cast<f32x4*>(lds);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int g = tid + 64 * NW * i;
      if ((NBLK * 64) % (64 * NW) == 0 || g < NBLK * 64) hl[slot(g >> 6, (g >> 2) & 15, g & 3)] = stage[i];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < RPT; ++j) hreg[j] = hl[strip(j)];
    transpose_groups();
  }
  __syncthreads();  // token vectors visible; packed H: LDS copy read before pb and part reuse it
  const f32x4 kq = *reinterpret_cast<const f32x4*>(&ks[4 * cq]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float kr = ks[row0 + i];
    f32x4 hv;
#pragma unroll
    for (int e = 0; e < 4; ++e) hv[e] = __builtin_fmaf(gam, hreg[i][e], bet * (kr * kq[e]));
    hreg[i] = hv;
    if constexpr (SYMH) {
      if (!mirror) __builtin_nontemporal_store(hv, Hp + myblk * 64 + (r0 + i) * 4 + cm);
    } else {
      __builtin_nontemporal_store(hv, at(Hb, i));
    }
  }

  // G's loads go out now and land during the solve: waiting for them after it
  // would leave every pair's G round trip exposed
  f32x4 greg[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) greg[i] = __builtin_nontemporal_load(at(Gb, i));
  // ---- CG on (H + Lambda) x = q -------------------------------------------------------
  if (lam_full) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) hreg[i] += lreg[i];
  }
  float xv[EPL], rv[EPL], pv[EPL], lv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) lv[e] = lam_full ? 0.f : lam_s[lane + 64 * e];
  float* mypb = pb[wave];
  // w = (H + Lambda) u for a vector u that every wave holds whole: this wave's
  // rows give column sums for all columns, the waves' parts meet in part2[buf]
  // at one barrier
  auto apply_a = [&](const float(&u)[EPL], float(&w)[EPL], int buf) {
    // publish u to this wave's own LDS copy (read back by the same wave only)
#pragma unroll
    for (int e = 0; e < EPL; ++e) mypb[lane + 64 * e] = u[e];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the writes above have landed
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i4 = 0; i4 < RPT / 4; ++i4) {
      const f32x4 pr = *reinterpret_cast<const f32x4*>(&mypb[row0 + 4 * i4]);
#pragma unroll
      for (int u4 = 0; u4 < 4; ++u4) acc += hreg[4 * i4 + u4] * pr[u4];
    }
    // combine the row groups of this wave: lanes l, l^32 (and l^16 when 4 groups)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (TPR == 4) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[e]), __float_as_uint(acc[e]), false, false);
        acc[e] = __uint_as_float(a[0]) + __uint_as_float(a[1]);
      }
      const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[e]), __float_as_uint(acc[e]), false, false);
      acc[e] = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    }
    float(*pt)[D] = part2[buf];
    if (lane < Q) *reinterpret_cast<f32x4*>(&pt[wave][4 * cq]) = acc;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int j = lane + 64 * e;
      float y = pt[0][j];
#pragma unroll
      for (int q = 1; q < NW; ++q) y += pt[q][j];
      w[e] = y + lv[e] * u[e];
    }
  };
  if constexpr (WARM) {
    // the part buffer used here is next written two barriers later
    float ax[EPL];
    apply_a(x0v, ax, 1);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      xv[e] = x0v[e];
      rv[e] = qs[lane + 64 * e] - ax[e];
      pv[e] = rv[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      xv[e] = 0.f;
      rv[e] = qs[lane + 64 * e];
      pv[e] = rv[e];
    }
  }
  // identical in every lane by construction; taken from lane 0 so that the
  // loop's exit tests are wave-uniform beyond doubt (a barrier is inside)
  auto vsum = [&](const float* a, const float* b) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) s += a[e] * b[e];
    return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(wave_sum(s))));
  };
  float rho = vsum(rv, rv);
  int n = 0;
  for (int it = 0; it < p.max_steps; ++it) {
    if (!(rho >= kCgZero && rho > p.tol2)) break;
    float wv[EPL];
    apply_a(pv, wv, it & 1);
    const float pw = vsum(pv, wv);
    if (!(pw >= kCgZero)) break;
    const float alpha = rho / pw;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      xv[e] += alpha * pv[e];
      rv[e] -= alpha * wv[e];
    }
    const float rr = vsum(rv, rv);
    const float bcg = rr / rho;
#pragma unroll
    for (int e = 0; e < EPL; ++e) pv[e] = rv[e] + bcg * pv[e];
    rho = rr;
    ++n;
  }
  // x to this wave's LDS copy for the G read-out
#pragma unroll
  for (int e = 0; e < EPL; ++e) mypb[lane + 64 * e] = xv[e];
  __builtin_amdgcn_s_waitcnt(0xc07f);

  // ---- G <- gamma G + beta (v k^T); o = G x ------------------------------------------
  const f32x4 xq = *reinterpret_cast<const f32x4*>(&mypb[4 * cq]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = row0 + i;
    const float bv = bet * vs[row];
    f32x4 gv;
#pragma unroll
    for (int e = 0; e < 4; ++e) gv[e] = __builtin_fmaf(gam, greg[i][e], bv * kq[e]);
    __builtin_nontemporal_store(gv, at(Gb, i));
    const float s = group_sum<Q>(gv[0] * xq[0] + gv[1] * xq[1] + gv[2] * xq[2] + gv[3] * xq[3]);
    if (cq == 0) p.o[(size_t)pair * D + row] = s;
  }
  if (wave == 0 && p.x_out) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) p.x_out[(size_t)pair * D + lane + 64 * e] = xv[e];
  }
  if (tid == 0 && p.steps) p.steps[pair] = n;
}

template <bool BF16, int D, bool SYMH, bool WARM>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<BF16, D, SYMH, WARM>), dim3(p.P), dim3(64 * kDecWaves), 0, s, p);
  return hipGetLastError();
}

template <bool SYMH, bool WARM>
hipError_t launch_decode_s(bool bf16, int D, const DecodeParams& p, hipStream_t s) {
  if (bf16) {
    if (D == 128) return launch_decode_t<true, 128, SYMH, WARM>(p, s);
    if (D == 64) return launch_decode_t<true, 64, SYMH, WARM>(p, s);
  } else {
    if (D == 128) return launch_decode_t<false, 128, SYMH, WARM>(p, s);
    if (D == 64) return launch_decode_t<false, 64, SYMH, WARM>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(bool bf16, int D, bool packed_h, bool warm, const DecodeParams& p, hipStream_t s) {
  if (packed_h) return warm ? launch_decode_s<true, true>(bf16, D, p, s) : launch_decode_s<true, false>(bf16, D, p, s);
  return warm ? launch_decode_s<false, true>(bf16, D, p, s) : launch_decode_s<false, false>(bf16, D, p, s);
}

}  // namespace mesa
