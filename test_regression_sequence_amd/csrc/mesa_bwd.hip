// Backward pass of the chunked Mesa layer by implicit differentiation of its
// solves (MesaNet page, technical summary, "Mesa layer": CG query response and
// chunk-parallel states; "architecture": the layer is trained end to end).
//
// With x_t the solution of (H_t + Lambda) x_t = q_t and o_t = G_t x_t, and
// d_o the gradient arriving at o:
//   dx_t = G_t^T d_o_t,            y_t = (H_t + Lambda)^{-1} dx_t   (adjoint solve)
//   dq_t = y_t,   local state gradients  dH_t = -y_t x_t^T,  dG_t = d_o_t x_t^T,
//   Hhat_t = dH_t + gamma_{t+1} Hhat_{t+1},  Ghat_t likewise (backward in time),
//   dk_t = beta_t ((Hhat_t + Hhat_t^T) k_t + Ghat_t^T v_t),   dv_t = beta_t Ghat_t k_t,
//   dbeta_t = k_t^T Hhat_t k_t + v_t^T Ghat_t k_t,   dlambda = -sum_t y_t * x_t.
// The forget factors: dgamma_t = <Hhat_t, H_{t-1}> + <Ghat_t, G_{t-1}>.  Inside a
// chunk with boundary states Hb, Gb and arriving adjoints Rb (of H; Rs = Rb + Rb^T)
// and S (of G), and b restarted at the chunk start s, gamma_t <Hhat_t, H_{t-1}> is
//   e^{b_e} <Rb, Hb>                                             (per chunk)
// + sum_{j<t} e^{b_e-b_j} beta_j k_j^T Rb k_j                     (prefix)
// + sum_{t'>=t} e^{b_t'} <dH_t', Hb>                               (suffix)
// + sum_{j<t<=t'} e^{b_t'-b_j} beta_j <dH_t', k_j k_j^T>           (pairs)
// and gamma_t <Ghat_t, G_{t-1}> likewise.  Every term's decay runs from a
// written token j < t past t, so it carries gamma_t and the division by
// gamma_t only rescales; every factor is a decay <= 1 and nothing accumulates
// across chunks (a cumulative sum of dL/db over the whole sequence would
// cancel to O(1) out of O(T) terms).
//
// Kernels (chunks of C = 64 tokens; s..e the chunk, b restarted at s):
//   bwd_dx_kernel    per chunk: dx = Gamma (d_O Gb) + (W o (d_O V^T)) K with
//                    W_tj = e^{b_t-b_j} beta_j [j<=t]; writes dx/||dx|| (bf16)
//                    and ||dx||, the right-hand sides of the adjoint CG (the
//                    forward CG kernels without their read-out; normalised
//                    right-hand sides make the stopping test relative).
//   bwd_scan_kernel  per stripe of 32 state rows of a sequence, chunks
//                    backwards (the next chunk's x, y, d_o loaded while the
//                    current one's products run): the adjoints arriving at a
//                    chunk's end, Rs = Hhat + Hhat^T and S = Ghat, stored per
//                    chunk (bf16), then
//                    Rs <- e^{b_e} Rs - sum_t w_t (y_t x_t^T + x_t y_t^T),
//                    S  <- e^{b_e} S + sum_t w_t d_o_t x_t^T,  w_t = e^{b_t};
//                    the final values give dh0 = Rs/2 and dg0 = S.  The
//                    update is linear in (Rs, S), so a long sequence is
//                    walked in segments: totals from zero, a carry pass
//                    (bwd_carry_kernel), then each segment from its carry-in.
//   bwd_scan_full_kernel  the same walk for many sequences: two workgroups per
//                    sequence, each holding half the rows of both Rs and S.
//   bwd_grad_kernel  per chunk: Hhat_t, Ghat_t applied to k_t, v_t as
//                    e^{b_e-b_t} (stored adjoint) k_t plus the chunk's own
//                    reverse-causal terms, e.g. Ghat_t k_t gains
//                    sum_{t'>=t} e^{b_t'-b_t} (x_t'.k_t) d_o_t'; the four parts of
//                    dgamma above; writes dq, dk, dv, dbeta, dgamma.
//   bwd_lambda_kernel dlambda summed over the batch (the scan sums each
//                    sequence's -y_t * x_t while staging its chunks).
//   bwd_lamfull_*    a full Lambda: dLambda = -sum_{b,t} y_t x_t^T per head,
//                    the partial derivative of each entry of the solves' matrix
//                    (fp32 products over 64-row tiles staged in LDS, in row
//                    splits, then the splits summed).
// Every chunk product is an MFMA 16x16x32 bf16 contraction with fp32
// accumulation on tiles staged in LDS with the contraction index contiguous
// (rows padded by 16 bytes, so the 16 rows an MFMA operand reads fall in
// distinct banks); fp32 inputs (x, y, d_o) are rounded to bf16 for the
// products only.
#include "mesa_common.h"
#include "mesa_kernels.h"

namespace mesa {

namespace {

constexpr int kC = 64;          // tokens per chunk
constexpr int kThreads = 256;   // 4 waves

__device__ __forceinline__ uint16_t bf(float x) { return __builtin_bit_cast(uint16_t, f32_to_bf16(x)); }

// 4x4 transpose inside each lane quad by two DPP butterfly stages: lane b of a
// quad holding x[i] = M[b][i] returns M[i][b].  Applied to an MFMA result tile
// (a lane's 4 rows of one column), it gives a lane 4 consecutive columns of
// one row, so the tile goes out as one 8-byte store per lane.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x) {
  const int qb = threadIdx.x & 3;
  f32x4 y, z;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t = __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x[i ^ 1]), 0xB1, 0xF, 0xF, false));
    y[i] = ((i & 1) == (qb & 1)) ? x[i] : t;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t = __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(y[i ^ 2]), 0x4E, 0xF, 0xF, false));
    z[i] = ((i & 2) == (qb & 2)) ? y[i] : t;
  }
  return z;
}
__device__ __forceinline__ u16x4 bf4(f32x4 v) { return u16x4{bf(v[0]), bf(v[1]), bf(v[2]), bf(v[3])}; }

// acc (16x16 tile; lane l holds rows 4(l/16)+{0..3} of column l%16) +=
// A[16][K] * Bt[16][K]^T, both bf16 in LDS with row strides lda, ldb.
template <int K>
__device__ __forceinline__ f32x4 mma(const uint16_t* A, int lda, const uint16_t* Bt, int ldb, f32x4 acc) {
  const int tl = threadIdx.x & 15, g = (threadIdx.x >> 4) & 3;
#pragma unroll
  for (int kb = 0; kb < K / 32; ++kb) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + tl * lda + 32 * kb + 8 * g);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bt + tl * ldb + 32 * kb + 8 * g);
    acc = mfma_bf16(a, b, acc);
  }
  return acc;
}

// b_t (inclusive prefix of log gamma from the chunk start) and beta_t of a
// chunk into LDS; tokens past Lc get gamma = 1, beta = 0.  Called by wave 0.
__device__ __forceinline__ void chunk_gates(const float* gamma, const float* beta, size_t row0, int Lc,
                                            float* bcum, float* betas) {
  const int lane = threadIdx.x & 63;
  float lg = 0.f, bt = 0.f;
  if (lane < Lc) {
    lg = logf(gamma[row0 + lane]);
    bt = beta[row0 + lane];
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(lg, o, 64);
    if (lane >= o) lg += t;
  }
  bcum[lane] = lg;
  betas[lane] = bt;
}

// Transposed staging: 8 neighbouring lanes take 8 consecutive tokens of one
// group of dims, so their LDS writes form 16-byte runs of a row (at most
// 2-way bank conflicts), while a wave instruction still reads 8 token rows x
// 128 contiguous bytes.  Thread mapping for quads (Q = D/4 groups of 4 dims):
// quad (tid/8) % Q, tokens tid%8 + 8 (blk + (32/Q) it), blk = (tid/8) / Q.
template <int D>
struct ColMap {
  static constexpr int Q = D / 4, BLKS = 32 / Q, N = kC * Q / kThreads;
  __device__ static int quad() { return (threadIdx.x >> 3) % Q; }
  __device__ static int tok(int it) { return (threadIdx.x & 7) + 8 * ((threadIdx.x >> 3) / Q + BLKS * it); }
};

// Split staging: the load halves return registers, so a kernel issues the loads
// of every tile it needs (or of a later phase) at once and writes LDS
// afterwards -- one memory round trip instead of one per tile.  Rows past Lc
// load row Lc-1 (every load is unconditional) and are written as zeros.
template <int D>
struct TileF32 { f32x4 v[kC * D / 4 / kThreads]; };
template <int D>
struct TileB16 { u16x8 v[kC * D / 8 / kThreads]; };
template <int D>
struct Square { u16x8 v[D * D / 8 / kThreads]; };

template <int D>
__device__ __forceinline__ TileF32<D> load_tile_f32(const float* src, int Lc) {
  constexpr int Q = D / 4;
  TileF32<D> r;
  const int c4 = threadIdx.x % Q, t0 = threadIdx.x / Q;
#pragma unroll
  for (int it = 0; it < kC * Q / kThreads; ++it)
    r.v[it] = *reinterpret_cast<const f32x4*>(src + (size_t)min(t0 + it * (kThreads / Q), Lc - 1) * D + 4 * c4);
  return r;
}
template <int D>
__device__ __forceinline__ void put_tile_f32(uint16_t* dst, int ld, const TileF32<D>& r, int Lc) {
  constexpr int Q = D / 4;
  const int c4 = threadIdx.x % Q, t0 = threadIdx.x / Q;
#pragma unroll
  for (int it = 0; it < kC * Q / kThreads; ++it) {
    const int t = t0 + it * (kThreads / Q);
    const float sc = t < Lc ? 1.f : 0.f;
    u16x4 o;
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = bf(r.v[it][u] * sc);
    *reinterpret_cast<u16x4*>(dst + t * ld + 4 * c4) = o;
  }
}
template <int D>
__device__ __forceinline__ TileB16<D> load_tile_b16(const uint16_t* src, int Lc) {
  constexpr int E = D / 8;
  TileB16<D> r;
  const int c8 = threadIdx.x % E, t0 = threadIdx.x / E;
#pragma unroll
  for (int it = 0; it < kC * E / kThreads; ++it)
    r.v[it] = *reinterpret_cast<const u16x8*>(src + (size_t)min(t0 + it * (kThreads / E), Lc - 1) * D + 8 * c8);
  return r;
}
template <int D>
__device__ __forceinline__ void put_tile_b16(uint16_t* dst, int ld, const TileB16<D>& r, int Lc) {
  constexpr int E = D / 8;
  const int c8 = threadIdx.x % E, t0 = threadIdx.x / E;
#pragma unroll
  for (int it = 0; it < kC * E / kThreads; ++it) {
    const int t = t0 + it * (kThreads / E);
    const u16x8 zero = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    *reinterpret_cast<u16x8*>(dst + t * ld + 8 * c8) = t < Lc ? r.v[it] : zero;
  }
}
template <int D>
__device__ __forceinline__ Square<D> load_square(const uint16_t* src) {
  Square<D> r;
#pragma unroll
  for (int it = 0; it < D * D / 8 / kThreads; ++it)
    r.v[it] = *reinterpret_cast<const u16x8*>(src + (size_t)(threadIdx.x + it * kThreads) * 8);
  return r;
}
// a boundary snapshot in fragment order into LDS row-major [D][ld]
template <int D>
__device__ __forceinline__ void put_frag(uint16_t* dst, int ld, const Square<D>& r) {
  constexpr int NM = D / 32;
#pragma unroll
  for (int it = 0; it < D * D / 8 / kThreads; ++it) {
    const int idx = threadIdx.x + it * kThreads;
    const int f = idx >> 6, l = idx & 63;
    const int n = 16 * (f / NM) + (l & 15);
    const int c0 = 32 * (f % NM) + 4 * (l >> 4);
    *reinterpret_cast<u16x4*>(dst + n * ld + c0) = u16x4{r.v[it][0], r.v[it][1], r.v[it][2], r.v[it][3]};
    *reinterpret_cast<u16x4*>(dst + n * ld + c0 + 16) = u16x4{r.v[it][4], r.v[it][5], r.v[it][6], r.v[it][7]};
  }
}
// the same, transposed: LDS [D][ld] holding the square's columns as rows
template <int D>
__device__ __forceinline__ void put_frag_t(uint16_t* dst, int ld, const Square<D>& r) {
  constexpr int NM = D / 32;
#pragma unroll
  for (int it = 0; it < D * D / 8 / kThreads; ++it) {
    const int idx = threadIdx.x + it * kThreads;
    const int f = idx >> 6, l = idx & 63;
    const int n = 16 * (f / NM) + (l & 15);
    const int c0 = 32 * (f % NM) + 4 * (l >> 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      dst[(c0 + u) * ld + n] = r.v[it][u];
      dst[(c0 + 16 + u) * ld + n] = r.v[it][4 + u];
    }
  }
}
// token-major [C][D] bf16 -> LDS transposed [D][ld] (octets of 8 dims): 8
// neighbouring lanes take 8 consecutive tokens of one octet, so their LDS
// writes form 16-byte runs of a row (at most 2-way bank conflicts), while a
// wave instruction still reads 8 token rows x 128 contiguous bytes
template <int D>
__device__ __forceinline__ int cols_tok(int it) {
  constexpr int E = D / 8, BLKS = 32 / E;
  return (threadIdx.x & 7) + 8 * ((threadIdx.x >> 3) / E + BLKS * it);
}
template <int D>
__device__ __forceinline__ TileB16<D> load_cols_b16(const uint16_t* src, int Lc) {
  constexpr int E = D / 8;
  TileB16<D> r;
  const int c8 = (threadIdx.x >> 3) % E;
#pragma unroll
  for (int it = 0; it < kC * E / kThreads; ++it)
    r.v[it] = *reinterpret_cast<const u16x8*>(src + (size_t)min(cols_tok<D>(it), Lc - 1) * D + 8 * c8);
  return r;
}
template <int D>
__device__ __forceinline__ void put_cols_b16(uint16_t* dst, int ld, const TileB16<D>& r, int Lc) {
  constexpr int E = D / 8;
  const int c8 = (threadIdx.x >> 3) % E;
#pragma unroll
  for (int it = 0; it < kC * E / kThreads; ++it) {
    const int t = cols_tok<D>(it);
#pragma unroll
    for (int u = 0; u < 8; ++u) dst[(8 * c8 + u) * ld + t] = t < Lc ? r.v[it][u] : uint16_t(0);
  }
}

// The adjoint snapshots Rs and S are stored in tile order: the 16x16 tile
// (mt, nt) of a square is 512 contiguous bytes, lane l of it 8 bytes holding
// row 16mt + 4(l/16) + l%4, columns 16nt + 4((l%16)/4) + {0..3} -- an MFMA
// result tile after quad_transpose -- so the adjoint scan stores whole tiles
// with one contiguous wave store each.  A 16-byte piece idx (as load_square
// reads it) is lanes 2(idx%32) and 2(idx%32)+1 of tile idx/32: rows r and r+1
// of one 4-column group.
__device__ __forceinline__ size_t adj_tile_offset(int D, int mt, int nt, int lane) {
  return ((size_t)(mt * (D / 16) + nt) * 64 + lane) * 4;
}
template <int D>
__device__ __forceinline__ void adj_piece(int idx, int& row, int& col) {
  const int u = idx >> 5, l0 = 2 * (idx & 31);
  const int tl = l0 & 15, g = l0 >> 4;
  row = 16 * (u / (D / 16)) + 4 * g + (tl & 3);
  col = 16 * (u % (D / 16)) + 4 * (tl >> 2);
}
// a tile-order square into LDS [D][ld], row-major (TRANS: transposed)
template <int D, bool TRANS>
__device__ __forceinline__ void put_adj(uint16_t* dst, int ld, const Square<D>& r) {
#pragma unroll
  for (int it = 0; it < D * D / 8 / kThreads; ++it) {
    int row, col;
    adj_piece<D>(threadIdx.x + it * kThreads, row, col);
    if constexpr (TRANS) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dst[(col + u) * ld + row] = r.v[it][u];
        dst[(col + u) * ld + row + 1] = r.v[it][4 + u];
      }
    } else {
      *reinterpret_cast<u16x4*>(dst + row * ld + col) = u16x4{r.v[it][0], r.v[it][1], r.v[it][2], r.v[it][3]};
      *reinterpret_cast<u16x4*>(dst + (row + 1) * ld + col) = u16x4{r.v[it][4], r.v[it][5], r.v[it][6], r.v[it][7]};
    }
  }
}
// <A, B> for a tile-order square held in registers and a row-major one in LDS [D][ld];
// this thread's part
template <int D>
__device__ __forceinline__ float dot_adj(const Square<D>& a, const uint16_t* b, int ld) {
  float acc = 0.f;
#pragma unroll
  for (int it = 0; it < D * D / 8 / kThreads; ++it) {
    int row, col;
    adj_piece<D>(threadIdx.x + it * kThreads, row, col);
    const u16x4 w0 = *reinterpret_cast<const u16x4*>(b + row * ld + col);
    const u16x4 w1 = *reinterpret_cast<const u16x4*>(b + (row + 1) * ld + col);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc = __builtin_fmaf(bf16_to_f32(a.v[it][u]), bf16_to_f32(w0[u]), acc);
      acc = __builtin_fmaf(bf16_to_f32(a.v[it][4 + u]), bf16_to_f32(w1[u]), acc);
    }
  }
  return acc;
}

// ---------------------------------------------------------------------------------------
// dx_t = G_t^T d_o_t, normalised right-hand sides of the adjoint solves
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dx_kernel(BwdParams p) {
  constexpr int LD = D + 8, LC = kC + 8, NTL = D / 16;
  constexpr int REG = (D * LD + kC * LD) > (kC * LC + D * LC) ? (D * LD + kC * LD) : (kC * LC + D * LC);
  const int chunk = blockIdx.x, bh = chunk / p.NC, c = chunk % p.NC;
  const int s = c * kC, Lc = min(kC, p.T - s);
  const size_t row0 = (size_t)bh * p.T + s;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, tl = lane & 15, g = lane >> 4;

  __shared__ float bcum[kC], betas[kC];
  __shared__ __attribute__((aligned(16))) uint16_t sDO[kC * LD];
  __shared__ __attribute__((aligned(16))) uint16_t sR[REG];
  uint16_t* sGT = sR;               // Gb^T  [D][LD]
  uint16_t* sV = sR + D * LD;       // V     [C][LD]
  uint16_t* sS = sR;                // masked scores [C][LC]  (after Gb^T, V are consumed)
  uint16_t* sKT = sR + kC * LC;     // K^T   [D][LC]

  // every global load of the chunk at once: d_O, V, Gb, and K for the second
  // product (held in registers until its LDS region is free)
  const TileF32<D> dov = load_tile_f32<D>(p.d_o + row0 * D, Lc);
  const TileB16<D> vv = load_tile_b16<D>(static_cast<const uint16_t*>(p.v) + row0 * D, Lc);
  const Square<D> gbv = load_square<D>(static_cast<const uint16_t*>(p.gb) + (size_t)chunk * D * D);
  const TileB16<D> kv = load_cols_b16<D>(static_cast<const uint16_t*>(p.k) + row0 * D, Lc);
  if (wave == 0) chunk_gates(p.gamma, p.beta, row0, Lc, bcum, betas);
  put_tile_f32<D>(sDO, LD, dov, Lc);
  put_tile_b16<D>(sV, LD, vv, Lc);
  put_frag_t<D>(sGT, LD, gbv);
  __syncthreads();

  f32x4 u[NTL], pp[4];
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt)
    u[nt] = mma<D>(sDO + 16 * wave * LD, LD, sGT + 16 * nt * LD, LD, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
    pp[jt] = mma<D>(sDO + 16 * wave * LD, LD, sV + 16 * jt * LD, LD, f32x4{0.f, 0.f, 0.f, 0.f});
  __syncthreads();  // Gb^T and V consumed
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * wave + 4 * g + i, j = 16 * jt + tl;
      const float w = j <= t ? expf(bcum[t] - bcum[j]) * betas[j] : 0.f;
      sS[t * LC + j] = bf(pp[jt][i] * w);
    }
  put_cols_b16<D>(sKT, LC, kv, Lc);
  __syncthreads();

  f32x4 r[NTL];
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt)
    r[nt] = mma<kC>(sS + 16 * wave * LC, LC, sKT + 16 * nt * LC, LC, f32x4{0.f, 0.f, 0.f, 0.f});

  uint16_t* rhs = static_cast<uint16_t*>(p.rhs);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * wave + 4 * g + i;
    const float gt = expf(bcum[t]);
    float ss = 0.f;
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
      r[nt][i] = __builtin_fmaf(gt, u[nt][i], r[nt][i]);
      ss = __builtin_fmaf(r[nt][i], r[nt][i], ss);
    }
    ss = group_sum<16>(ss);
    const float nrm = sqrtf(ss);
    const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) r[nt][i] *= inv;
    if (t < Lc && tl == 0) p.nu[row0 + t] = nrm;
  }
  // token 16 wave + 4g + (lane quad position), dims 16nt + 4(tl/4) + {0..3}
  const int tq = 16 * wave + 4 * g + (tl & 3);
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt) {
    const f32x4 z = quad_transpose(r[nt]);
    if (tq < Lc) *reinterpret_cast<u16x4*>(rhs + (row0 + tq) * D + 16 * nt + (tl & ~3)) = bf4(z);
  }
}

// ---------------------------------------------------------------------------------------
// adjoint scan, chunks backwards; a workgroup owns a stripe of 32 state rows of one
// sequence segment.  With TOTALS it walks segment s >= 1 from a zero state and leaves
// the segment's total and decay for the carry pass; otherwise it walks segment s from
// its carry-in state (the final-state adjoint for the last segment), storing snapshots.
// ---------------------------------------------------------------------------------------
template <int D, bool TOTALS>
__global__ __launch_bounds__(kThreads) void bwd_scan_kernel(BwdParams p) {
  constexpr int SR = 32, NSTR = D / SR;          // state rows per workgroup, stripes per sequence
  constexpr int CW = D / 4, NCT = CW / 16;       // state columns per wave, their 16-column tiles
  constexpr int NRT = SR / 16;
  constexpr int L2 = 2 * kC + 8, LC = kC + 8;
  using M = ColMap<D>;                            // x, y: all dims; token-contiguous lane groups
  constexpr int Q = M::Q, NQ = M::N;
  constexpr int SQ = SR / 4, ND = kC * SQ / kThreads;  // d_o: the stripe's dims
  static_assert(ND >= 1 && ND * kThreads == kC * SQ, "stripe items per thread");
  // XCD-aware decode: the stripes of one (sequence, segment) share blockIdx % 8 and are
  // dispatched side by side, so the chunk's x and y tiles they all read come through
  // one L2
  const int NSP = TOTALS ? p.NS - 1 : p.NS;  // segments walked by this launch
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int stripe = local % NSTR, r0 = SR * stripe;
  const int sg = (local / NSTR) % NSP + (TOTALS ? 1 : 0);
  const int bh = (local / NSTR / NSP) * 8 + xcd;
  if (bh >= p.BH) return;
  const int cb = sg * p.SEG, ce = min(cb + p.SEG, p.NC);  // this segment's chunks
  const size_t D2 = (size_t)D * D;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, tl = lane & 15, g = lane >> 4;
  const int qc = M::quad();                                        // this thread's dim quad
  const bool own = 4 * qc >= r0 && 4 * qc < r0 + SR;               // quad inside the stripe
  const int dq = (threadIdx.x >> 3) % SQ;                          // d_o: stripe quad
  auto dtok = [&](int it) { return (threadIdx.x & 7) + 8 * ((threadIdx.x >> 3) / SQ + (kThreads / 8 / SQ) * it); };

  __shared__ __attribute__((aligned(16))) uint16_t sA1[SR * L2];  // [(-wY)^T | (-wX)^T], stripe rows
  __shared__ __attribute__((aligned(16))) uint16_t sB1[D * L2];   // [X^T | Y^T], all dims
  __shared__ __attribute__((aligned(16))) uint16_t sA2[SR * LC];  // (w d_O)^T, stripe rows
  __shared__ __attribute__((aligned(16))) f32x4 lam_s[kThreads];

  // start state: zero for a segment total, the final-state adjoint for the last
  // segment, the carry-in state for an earlier one
  const bool from_final = !TOTALS && sg == p.NS - 1;
  const float* carry_r = (!TOTALS && !from_final) ? p.seg_state + (((size_t)bh * 2) * (p.NS - 1) + sg) * D2 : nullptr;
  const float* carry_s = carry_r ? carry_r + (size_t)(p.NS - 1) * D2 : nullptr;
  // (the sources are chosen per workgroup, so each batch of loads is issued at once)
  const float* src_r = from_final ? (p.d_hfinal ? p.d_hfinal + (size_t)bh * D2 : nullptr) : carry_r;
  const float* src_s = from_final ? (p.d_gfinal ? p.d_gfinal + (size_t)bh * D2 : nullptr) : carry_s;
  f32x4 R[NRT][NCT], S[NRT][NCT];
  auto load_square_part = [&](const float* src, bool transposed, f32x4 (&dst)[NRT][NCT]) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int row = r0 + 16 * rt + 4 * g + ii, col = CW * wave + 16 * ct + tl;
          dst[rt][ct][ii] = transposed ? src[col * D + row] : src[row * D + col];
        }
  };
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      R[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      S[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  if (src_r) load_square_part(src_r, false, R);
  if (src_s) load_square_part(src_s, false, S);
  if (from_final && src_r) {
    // the final-state adjoint of H enters symmetrised: D_h + D_h^T
    f32x4 T[NRT][NCT];
    load_square_part(src_r, true, T);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) R[rt][ct] += T[rt][ct];
  }

  // x, y (all dims), d_o (stripe dims) and the gates of a chunk, into registers
  f32x4 xv[NQ], yv[NQ], dv[ND];
  float gam_n = 1.f, nu_n = 0.f;  // one token per lane, in every wave
  auto fetch = [&](int c) {
    const int Lc = min(kC, p.T - c * kC);
    const size_t row0 = (size_t)bh * p.T + c * kC;
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const size_t r = row0 + min(M::tok(it), Lc - 1);
      xv[it] = *reinterpret_cast<const f32x4*>(p.x + r * D + 4 * qc);
      yv[it] = *reinterpret_cast<const f32x4*>(p.yn + r * D + 4 * qc);
    }
#pragma unroll
    for (int it = 0; it < ND; ++it) {
      const size_t r = row0 + min(dtok(it), Lc - 1);
      dv[it] = *reinterpret_cast<const f32x4*>(p.d_o + r * D + r0 + 4 * dq);
    }
    {
      const size_t r = row0 + min(lane, Lc - 1);
      gam_n = p.gamma[r];
      nu_n = p.nu[r];
    }
  };
  f32x4 lam = f32x4{0.f, 0.f, 0.f, 0.f};
  float logdec = 0.f;  // the segment's total log decay
  if (ce > cb) fetch(ce - 1);

  for (int c = ce - 1; c >= cb; --c) {
    const int chunk = bh * p.NC + c;
    const int s = c * kC, Lc = min(kC, p.T - s);
    if constexpr (!TOTALS) {
      // the adjoints arriving at this chunk's end, one 8-byte store per tile and lane
      uint16_t* snR = p.snap_r + (size_t)chunk * D2;
      uint16_t* snS = p.snap_s + (size_t)chunk * D2;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const size_t o = adj_tile_offset(D, r0 / 16 + rt, (CW * wave) / 16 + ct, lane);
          *reinterpret_cast<u16x4*>(snR + o) = bf4(quad_transpose(R[rt][ct]));
          *reinterpret_cast<u16x4*>(snS + o) = bf4(quad_transpose(S[rt][ct]));
        }
    }
    // the gates, in every wave (lane = token): no barrier between them and the staging
    float lg = lane < Lc ? logf(gam_n) : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_up(lg, o, 64);
      if (lane >= o) lg += t;
    }
    const float wt_l = expf(lg);
    const float nu_l = lane < Lc ? nu_n : 0.f;
    const float blast = __shfl(lg, 63, 64);  // the chunk's total log decay
    // y_t = nu_t * yn_t: X^T, Y^T into sB1; -(w Y)^T, -(w X)^T of the stripe into sA1;
    // stripe 0 also sums this thread's dims of dlambda = -sum_t y_t * x_t
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int t = M::tok(it);
      const bool in = t < Lc;
      const float wsh = __shfl(wt_l, t, 64), nsh = __shfl(nu_l, t, 64);
      const float w = in ? wsh : 0.f, nu = in ? nsh : 0.f, ex = in ? 1.f : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 4 * qc + u;
        const float xe = xv[it][u] * ex, ye = yv[it][u] * nu;
        sB1[i * L2 + t] = bf(xe);
        sB1[i * L2 + kC + t] = bf(ye);
        if (own) {
          sA1[(i - r0) * L2 + t] = bf(-w * ye);
          sA1[(i - r0) * L2 + kC + t] = bf(-w * xe);
        }
        if (!TOTALS && stripe == 0) lam[u] = __builtin_fmaf(-ye, xe, lam[u]);
      }
    }
#pragma unroll
    for (int it = 0; it < ND; ++it) {
      const int t = dtok(it);
      const float wsh = __shfl(wt_l, t, 64);
      const float w = t < Lc ? wsh : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) sA2[(4 * dq + u) * LC + t] = bf(w * dv[it][u]);
    }
    if (c > cb) fetch(c - 1);  // the next chunk's loads fly during this chunk's products
    __syncthreads();
    logdec += blast;
    const float decay = expf(blast);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint16_t* bt = sB1 + (CW * wave + 16 * ct) * L2;
        R[rt][ct] = mma<2 * kC>(sA1 + 16 * rt * L2, L2, bt, L2, R[rt][ct] * decay);
        S[rt][ct] = mma<kC>(sA2 + 16 * rt * LC, LC, bt, L2, S[rt][ct] * decay);
      }
    __syncthreads();
  }
  if constexpr (TOTALS) {
    // the segment's total from a zero start, and its decay, for the carry pass
    float* tr = p.seg_state + (((size_t)bh * 2) * (p.NS - 1) + sg - 1) * D2;
    float* ts = tr + (size_t)(p.NS - 1) * D2;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int row = r0 + 16 * rt + 4 * g + ii, col = CW * wave + 16 * ct + tl;
          tr[row * D + col] = R[rt][ct][ii];
          ts[row * D + col] = S[rt][ct][ii];
        }
    if (stripe == 0 && threadIdx.x == 0) p.seg_decay[(size_t)bh * (p.NS - 1) + sg - 1] = expf(logdec);
    return;
  }
  // this segment's part of dlambda: the threads sharing a dim quad
  if (stripe == 0) {
    lam_s[threadIdx.x] = lam;
    __syncthreads();
    if (threadIdx.x < Q) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int r = 0; r < kThreads; ++r)
        if (((r >> 3) % Q) == (int)threadIdx.x) acc += lam_s[r];
      *reinterpret_cast<f32x4*>(p.lam_part + ((size_t)bh * p.NS + sg) * D + 4 * threadIdx.x) = acc;
    }
  }
  // gradients of the initial states
  if (sg == 0) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int row = r0 + 16 * rt + 4 * g + ii, col = CW * wave + 16 * ct + tl;
          if (p.dh0) p.dh0[(size_t)bh * D2 + row * D + col] = 0.5f * R[rt][ct][ii];
          if (p.dg0) p.dg0[(size_t)bh * D2 + row * D + col] = S[rt][ct][ii];
        }
  }
}

// ---------------------------------------------------------------------------------------
// adjoint scan with whole states, for 2 BH >= 256 (one walk per sequence): two
// workgroups of 8 waves per sequence, each holding one half of the rows of both
// Rs and S.  The two do equal work and both read the chunk's x and y, so they
// walk at one pace and the second read of x and y hits in their shared L2 (the
// stripe walk above stages every chunk's x and y once per 32-row stripe).  Same
// products, in the same order, as the stripe walk: the snapshots and dh0, dg0
// are bitwise those of the stripe walk.
// ---------------------------------------------------------------------------------------
constexpr int kFullThreads = 512;

// the walk of one half (HF: rows HF*D/2 .. HF*D/2 + D/2 - 1) of both states
template <int D, int HF>
__device__ __forceinline__ void adj_full_walk(const BwdParams& p, int bh, uint16_t (*sB2)[D * (2 * kC + 8)],
                                              uint16_t (*sAR2)[(D / 2) * (2 * kC + 8)],
                                              uint16_t (*sAS2)[(D / 2) * (kC + 8)]) {
  constexpr int NW = kFullThreads / 64, ND = D / 16, NH = ND / 2;  // row tiles per half
  constexpr int UPW = NH * ND / NW;                   // tiles of each state per wave
  constexpr int L2 = 2 * kC + 8, LC = kC + 8;         // token blocks + 16 bytes of padding
  constexpr int NIT = (kC / 2) * (D / 4) / kFullThreads;  // (token pair, dim quad) items per thread
  constexpr int QH = D / 8;                           // dim quads per half
  static_assert(UPW * NW == NH * ND && NIT * kFullThreads == (kC / 2) * (D / 4), "whole tiles and items");
  // items of this half's dims: with D = 128 exactly item HF of every thread,
  // with D = 64 the one item of the threads whose quad lies in the half
  constexpr int NMI = NIT > 1 ? 1 : NIT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, tl = lane & 15, g = lane >> 4;
  const size_t D2 = (size_t)D * D;
  auto item_dq = [&](int it) { return (tid + kFullThreads * it) / (kC / 2); };
  auto mine_it = [&](int it) { return NIT > 1 ? it == HF : item_dq(it) / QH == HF; };
  constexpr int MIT = NIT > 1 ? HF : 0;               // the item slot that can be this half's

  // start state: the final-state adjoints (zero without them); lane (tl, g) of
  // tile u = (mt, nt) holds rows 16mt + 4g + i of column 16nt + tl, with
  // mt = HF * NH + u / ND (each batch of loads is issued at once)
  f32x4 R[UPW], S[UPW];
  auto tile_mt = [&](int ui) { return HF * NH + (wave + NW * ui) / ND; };
  auto tile_nt = [&](int ui) { return (wave + NW * ui) % ND; };
  auto load_tiles = [&](const float* F, bool transposed, f32x4 (&dst)[UPW]) {
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * tile_mt(ui) + 4 * g + i, col = 16 * tile_nt(ui) + tl;
        dst[ui][i] = transposed ? F[col * D + row] : F[row * D + col];
      }
    }
  };
#pragma unroll
  for (int ui = 0; ui < UPW; ++ui) {
    R[ui] = f32x4{0.f, 0.f, 0.f, 0.f};
    S[ui] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (p.d_hfinal) {
    // the final-state adjoint of H enters symmetrised: D_h + D_h^T
    const float* F = p.d_hfinal + (size_t)bh * D2;
    f32x4 T[UPW];
    load_tiles(F, false, R);
    load_tiles(F, true, T);
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) R[ui] += T[ui];
  }
  if (p.d_gfinal) load_tiles(p.d_gfinal + (size_t)bh * D2, false, S);

  // one chunk's inputs in registers: x and y / ||dx|| of this thread's items
  // (tokens 2jp, 2jp+1 x dims 4dq..4dq+3), d_o of its item in this half, and
  // one token's gates per lane
  struct Raw {
    f32x4 x[NIT][2], y[NIT][2], o[NMI][2];
    float gam, nu;
  };
  auto fetch = [&](int c, Raw& r) {
    const int Lc = min(kC, p.T - c * kC);
    const size_t row0 = (size_t)bh * p.T + c * kC;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int pc = tid + kFullThreads * it, jp = pc % (kC / 2), dq = pc / (kC / 2);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const size_t rr = row0 + min(2 * jp + h, Lc - 1);
        r.x[it][h] = *reinterpret_cast<const f32x4*>(p.x + rr * D + 4 * dq);
        r.y[it][h] = *reinterpret_cast<const f32x4*>(p.yn + rr * D + 4 * dq);
        if (it == MIT && mine_it(it)) r.o[0][h] = *reinterpret_cast<const f32x4*>(p.d_o + rr * D + 4 * dq);
      }
    }
    const size_t rl = row0 + min(lane, Lc - 1);
    r.gam = p.gamma[rl];
    r.nu = p.nu[rl];
  };
  f32x4 lam = f32x4{0.f, 0.f, 0.f, 0.f};

  // the adjoints arriving at chunk c's end, one 8-byte store per tile and lane
  auto store_snapshot = [&](const int c) {
    uint16_t* sr = p.snap_r + ((size_t)bh * p.NC + c) * D2;
    uint16_t* ss = p.snap_s + ((size_t)bh * p.NC + c) * D2;
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
      const size_t off = adj_tile_offset(D, tile_mt(ui), tile_nt(ui), lane);
      *reinterpret_cast<u16x4*>(sr + off) = bf4(quad_transpose(R[ui]));
      *reinterpret_cast<u16x4*>(ss + off) = bf4(quad_transpose(S[ui]));
    }
  };
  // chunk c from ring buffer cur, with chunk c-2 fetched into pre (two steps ahead).
  // LDS (this parity): sB = [X^T | Y^T] (all dims); sAR = [(-wY)^T | (-wX)^T] and
  // sAS = (w d_O)^T (this half's dims)
  auto step = [&](const int c, const Raw& cur, Raw& pre) {
    const int Lc = min(kC, p.T - c * kC);
    uint16_t* sB = sB2[c & 1];
    uint16_t* sAR = sAR2[c & 1];
    uint16_t* sAS = sAS2[c & 1];
    fetch(max(c - 2, 0), pre);  // unconditional (clamped): no branch among the loads
    // the gates (lane = token): w_t = e^{b_t}, b restarted at the chunk start
    float lg = lane < Lc ? logf(cur.gam) : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t = __shfl_up(lg, o, 64);
      if (lane >= o) lg += t;
    }
    const float wt_l = expf(lg);
    const float nu_l = lane < Lc ? cur.nu : 0.f;
    const float blast = __shfl(lg, 63, 64);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int pc = tid + kFullThreads * it, jp = pc % (kC / 2), dq = pc / (kC / 2);
      const int t0 = 2 * jp, t1 = t0 + 1;
      const float ws0 = __shfl(wt_l, t0, 64), ws1 = __shfl(wt_l, t1, 64);
      const float ns0 = __shfl(nu_l, t0, 64), ns1 = __shfl(nu_l, t1, 64);
      const bool in0 = t0 < Lc, in1 = t1 < Lc;
      const float w0 = in0 ? ws0 : 0.f, w1 = in1 ? ws1 : 0.f;
      const float ex0 = in0 ? 1.f : 0.f, ex1 = in1 ? 1.f : 0.f;
      const bool mine = it == MIT && mine_it(it);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 4 * dq + u, il = i - HF * (D / 2);
        const float xe0 = cur.x[it][0][u] * ex0, xe1 = cur.x[it][1][u] * ex1;
        const float ye0 = cur.y[it][0][u] * (in0 ? ns0 : 0.f), ye1 = cur.y[it][1][u] * (in1 ? ns1 : 0.f);
        *reinterpret_cast<uint32_t*>(sB + i * L2 + t0) = (uint32_t)bf(xe0) | ((uint32_t)bf(xe1) << 16);
        *reinterpret_cast<uint32_t*>(sB + i * L2 + kC + t0) = (uint32_t)bf(ye0) | ((uint32_t)bf(ye1) << 16);
        if (mine) {
          *reinterpret_cast<uint32_t*>(sAR + il * L2 + t0) =
              (uint32_t)bf(-w0 * ye0) | ((uint32_t)bf(-w1 * ye1) << 16);
          *reinterpret_cast<uint32_t*>(sAR + il * L2 + kC + t0) =
              (uint32_t)bf(-w0 * xe0) | ((uint32_t)bf(-w1 * xe1) << 16);
          *reinterpret_cast<uint32_t*>(sAS + il * LC + t0) =
              (uint32_t)bf(w0 * cur.o[0][0][u]) | ((uint32_t)bf(w1 * cur.o[0][1][u]) << 16);
          lam[u] = __builtin_fmaf(-ye0, xe0, lam[u]);
          lam[u] = __builtin_fmaf(-ye1, xe1, lam[u]);
        }
      }
    }
    // every wave finished chunk c+2's products, which read this parity's
    // buffers, before chunk c+1's barrier
    __syncthreads();
    const float decay = expf(blast);
#pragma unroll
    for (int ui = 0; ui < UPW; ++ui) {
      const int ml = tile_mt(ui) - HF * NH, nt = tile_nt(ui);
      R[ui] = mma<2 * kC>(sAR + 16 * ml * L2, L2, sB + 16 * nt * L2, L2, R[ui] * decay);
      S[ui] = mma<kC>(sAS + 16 * ml * LC, LC, sB + 16 * nt * L2, L2, S[ui] * decay);
    }
    // the adjoints arriving at chunk c-1's end go out now, so their stores drain
    // while the next chunk is gated and staged
    if (c > 0) store_snapshot(c - 1);
  };
  Raw b0, b1, b2;
  if (p.NC > 0) {
    store_snapshot(p.NC - 1);
    fetch(p.NC - 1, b0);
    fetch(max(p.NC - 2, 0), b1);
  }
  for (int c = p.NC - 1; c >= 0; c -= 3) {
    step(c, b0, b2);
    if (c - 1 >= 0) step(c - 1, b1, b0);
    if (c - 2 >= 0) step(c - 2, b2, b1);
  }

  // this sequence's part of dlambda over this half's dims: the 32 threads of a
  // dim quad are one half-wave
  {
    f32x4 sum;
#pragma unroll
    for (int u = 0; u < 4; ++u) sum[u] = group_sum<32>(lam[u]);
    if ((tid & 31) == 0 && mine_it(MIT))
      *reinterpret_cast<f32x4*>(p.lam_part + (size_t)bh * D + 4 * item_dq(MIT)) = sum;
  }
  // gradients of the initial states
#pragma unroll
  for (int ui = 0; ui < UPW; ++ui) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * tile_mt(ui) + 4 * g + i, col = 16 * tile_nt(ui) + tl;
      if (p.dh0) p.dh0[(size_t)bh * D2 + row * D + col] = 0.5f * R[ui][i];
      if (p.dg0) p.dg0[(size_t)bh * D2 + row * D + col] = S[ui][i];
    }
  }
}

template <int D>
__global__ __launch_bounds__(kFullThreads) void bwd_scan_full_kernel(BwdParams p) {
  // XCD-aware decode: the two workgroups of a sequence share blockIdx % 8, so the
  // chunk's x and y they both read come through one L2
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int half = local & 1;
  const int bh = (local >> 1) * 8 + xcd;
  if (bh >= p.BH) return;
  // double-buffered by chunk parity, so one barrier per chunk
  __shared__ __attribute__((aligned(16))) uint16_t sB2[2][D * (2 * kC + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sAR2[2][(D / 2) * (2 * kC + 8)];
  __shared__ __attribute__((aligned(16))) uint16_t sAS2[2][(D / 2) * (kC + 8)];
  if (half == 0) adj_full_walk<D, 0>(p, bh, sB2, sAR2, sAS2);
  else adj_full_walk<D, 1>(p, bh, sB2, sAR2, sAS2);
}

// Carry pass of a segmented adjoint scan, backwards over the segments: C_{NS-1} is the
// final-state adjoint and C_{s-1} = Gamma_s C_s + total_s, left in the slot where
// total_s was (the carry-in state of segment s-1).
__global__ __launch_bounds__(256) void bwd_carry_kernel(BwdParams p, int D) {
  const size_t D2 = (size_t)D * D;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)p.BH * 2 * (long long)D2) return;
  const int e = (int)(idx % D2), which = (int)((idx / D2) % 2);
  const int bh = (int)(idx / D2 / 2);
  const int row = e / D, col = e % D;
  float c = 0.f;
  if (which == 0 && p.d_hfinal) c = p.d_hfinal[bh * D2 + row * D + col] + p.d_hfinal[bh * D2 + col * D + row];
  if (which == 1 && p.d_gfinal) c = p.d_gfinal[bh * D2 + e];
  for (int sg = p.NS - 1; sg >= 1; --sg) {
    float* t = p.seg_state + (((size_t)bh * 2 + which) * (p.NS - 1) + sg - 1) * D2 + e;
    c = __builtin_fmaf(p.seg_decay[(size_t)bh * (p.NS - 1) + sg - 1], c, *t);
    *t = c;
  }
}

// ---------------------------------------------------------------------------------------
// per-token gradients of a chunk
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_grad_kernel(BwdParams p) {
  constexpr int LD = D + 8, L2 = 2 * kC + 8, LC = kC + 8, NTL = D / 16;
  constexpr int R1A = 5 * kC * LD;                       // K, V, X, Y, d_O token-major
  constexpr int R1B = 2 * kC * LD + D * L2 + D * LC;     // K, V, [Y^T | X^T], d_O^T
  constexpr int R1 = R1A > R1B ? R1A : R1B;
  const int chunk = blockIdx.x, bh = chunk / p.NC, c = chunk % p.NC;
  const int h = bh % p.H;
  const int s = c * kC, Lc = min(kC, p.T - s);
  const size_t row0 = (size_t)bh * p.T + s;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, tl = lane & 15, g = lane >> 4;

  __shared__ float bcum[kC], betas[kC], nus[kC];
  __shared__ float ta[kC], tsuf[kC], trs[kC], tcol[4][kC];  // dgamma parts per token
  __shared__ float red[2][4];                                          // <Rs, Hb>, <S, Gb> per wave
  __shared__ __attribute__((aligned(16))) uint16_t r1[R1];
  __shared__ __attribute__((aligned(16))) uint16_t r2[D * LD];          // Hb, Gb, then Rs, S, S^T
  __shared__ __attribute__((aligned(16))) uint16_t r3[kC * L2 + kC * LC];  // scores
  uint16_t* sK = r1;
  uint16_t* sV = r1 + kC * LD;
  uint16_t* sX = r1 + 2 * kC * LD;
  uint16_t* sY = r1 + 3 * kC * LD;
  uint16_t* sDO = r1 + 4 * kC * LD;
  uint16_t* sYX = r1 + 2 * kC * LD;             // [Y^T | X^T]  (after the scores)
  uint16_t* sDOT = sYX + D * L2;                // d_O^T
  uint16_t* sA3 = r3;                           // [-M o Pxk | -M o Pyk]
  uint16_t* sMvd = r3 + kC * L2;                // M o Pvd
  const size_t sn = (size_t)chunk * D * D;

  // ---- every load of the first phase at once; wave 0 forms the gates meanwhile ----------
  const TileB16<D> kt = load_tile_b16<D>(static_cast<const uint16_t*>(p.k) + row0 * D, Lc);
  const TileB16<D> vt = load_tile_b16<D>(static_cast<const uint16_t*>(p.v) + row0 * D, Lc);
  const TileF32<D> xt = load_tile_f32<D>(p.x + row0 * D, Lc);
  const TileF32<D> yt = load_tile_f32<D>(p.yn + row0 * D, Lc);   // y / ||dx||: scaled where used
  const TileF32<D> dt = load_tile_f32<D>(p.d_o + row0 * D, Lc);
  const Square<D> hbs = load_square<D>(static_cast<const uint16_t*>(p.hb) + sn);
  if (wave == 0) {
    chunk_gates(p.gamma, p.beta, row0, Lc, bcum, betas);
    nus[lane] = lane < Lc ? p.nu[row0 + lane] : 0.f;
  }
  put_tile_b16<D>(sK, LD, kt, Lc);
  put_tile_b16<D>(sV, LD, vt, Lc);
  put_tile_f32<D>(sX, LD, xt, Lc);
  put_tile_f32<D>(sY, LD, yt, Lc);
  put_tile_f32<D>(sDO, LD, dt, Lc);
  put_frag<D>(r2, LD, hbs);
  __syncthreads();
  // dq = y
  {
    constexpr int Q = D / 4;
    const int c4 = threadIdx.x % Q, t0 = threadIdx.x / Q;
#pragma unroll
    for (int it = 0; it < kC * Q / kThreads; ++it) {
      const int t = t0 + it * (kThreads / Q);
      if (t < Lc) *reinterpret_cast<f32x4*>(p.dq + (row0 + t) * D + 4 * c4) = yt.v[it] * nus[t];
    }
  }

  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  const int trow = 16 * wave;
  // ---- dgamma: suffix terms e^{b_t}(<dH_t, Hb> + <dG_t, Gb>) and the per-chunk ones ------
  const Square<D> gbs = load_square<D>(static_cast<const uint16_t*>(p.gb) + sn);  // next phase
  const Square<D> rss = load_square<D>(p.snap_r + sn);                             // Rs: <Rs, Hb>, then staged
  const Square<D> sqs = load_square<D>(p.snap_s + sn);                             // S: <S, Gb>, then staged
  float cpart[4];
  {
    f32x4 hx[NTL];
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) hx[nt] = mma<D>(sX + trow * LD, LD, r2 + 16 * nt * LD, LD, z);  // Hb x_t
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = trow + 4 * g + i;
      float a = 0.f;
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) a = __builtin_fmaf(bf16_to_f32(sY[t * LD + 16 * nt + tl]), hx[nt][i], a);
      cpart[i] = -nus[t] * a;  // <dH_t, Hb> = -y_t^T Hb x_t
    }
    const float rh = wave_sum(dot_adj<D>(rss, r2, LD));
    if (lane == 0) red[0][wave] = rh;
  }
  __syncthreads();  // Hb consumed
  put_frag<D>(r2, LD, gbs);
  __syncthreads();
  {
    f32x4 gx[NTL];
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) gx[nt] = mma<D>(sX + trow * LD, LD, r2 + 16 * nt * LD, LD, z);  // Gb x_t
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = trow + 4 * g + i;
      float a = 0.f;
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) a = __builtin_fmaf(bf16_to_f32(sDO[t * LD + 16 * nt + tl]), gx[nt][i], a);
      const float tot = group_sum<16>(cpart[i] + a);  // + <dG_t, Gb> = d_o_t^T Gb x_t
      if (tl == 0) tsuf[t] = t < Lc ? expf(bcum[t]) * tot : 0.f;
    }
    const float sg = wave_sum(dot_adj<D>(sqs, r2, LD));
    if (lane == 0) red[1][wave] = sg;
  }
  // ---- reverse-causal scores (t' >= t), masked and decayed ----------------------------
  {
    f32x4 pxk[4], pyk[4], pvd[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      pxk[jt] = mma<D>(sK + trow * LD, LD, sX + 16 * jt * LD, LD, z);   // k_t . x_t'
      pyk[jt] = mma<D>(sK + trow * LD, LD, sY + 16 * jt * LD, LD, z);   // k_t . y_t' / ||dx_t'||
      pvd[jt] = mma<D>(sV + trow * LD, LD, sDO + 16 * jt * LD, LD, z);  // v_t . d_o_t'
    }
    // pairs j <= t': e^{b_t'-b_j} beta_j (<dH_t', k_j k_j^T> + <dG_t', v_j k_j^T>), row sums and column sums
    float rowacc[4] = {0.f, 0.f, 0.f, 0.f}, colacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = trow + 4 * g + i, tp = 16 * jt + tl;
        const float m = tp >= t ? expf(bcum[tp] - bcum[t]) : 0.f;
        pyk[jt][i] *= nus[tp];
        sA3[t * L2 + tp] = bf(-m * pxk[jt][i]);
        sA3[t * L2 + kC + tp] = bf(-m * pyk[jt][i]);
        sMvd[t * LC + tp] = bf(m * pvd[jt][i]);
        const float e = m * betas[t] * pxk[jt][i] * (pvd[jt][i] - pyk[jt][i]);
        rowacc[i] += e;
        colacc[jt] += e;
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float r = group_sum<16>(rowacc[i]);
      if (tl == 0) trs[trow + 4 * g + i] = r;
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const float cs = sum_lane_groups(colacc[jt]);
      if (g == 0) tcol[wave][16 * jt + tl] = cs;
    }
  }
  // the transposed tiles come from the token-major ones in LDS: read here, written
  // over them after the barrier
  using CM = ColMap<D>;
  u16x4 ycol[CM::N], xcol[CM::N], dcol[CM::N];
#pragma unroll
  for (int it = 0; it < CM::N; ++it) {
    const int o = CM::tok(it) * LD + 4 * CM::quad();
    ycol[it] = *reinterpret_cast<const u16x4*>(sY + o);
    xcol[it] = *reinterpret_cast<const u16x4*>(sX + o);
    dcol[it] = *reinterpret_cast<const u16x4*>(sDO + o);
  }
  __syncthreads();  // X, Y, d_O token-major and Gb consumed
  // ---- stored adjoints of the chunk's end, applied to k_t and v_t ---------------------
  put_adj<D, false>(r2, LD, rss);
#pragma unroll
  for (int it = 0; it < CM::N; ++it) {
    const int t = CM::tok(it), i0 = 4 * CM::quad();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sYX[(i0 + u) * L2 + t] = bf(nus[t] * bf16_to_f32(ycol[it][u]));  // Y^T
      sYX[(i0 + u) * L2 + kC + t] = xcol[it][u];                        // X^T
      sDOT[(i0 + u) * LC + t] = dcol[it][u];                            // d_O^T
    }
  }
  __syncthreads();
  f32x4 hk[NTL], gk[NTL], gtv[NTL];
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt) hk[nt] = mma<D>(sK + trow * LD, LD, r2 + 16 * nt * LD, LD, z);
  __syncthreads();
  put_adj<D, false>(r2, LD, sqs);
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt) gk[nt] = mma<D>(sK + trow * LD, LD, r2 + 16 * nt * LD, LD, z);
  __syncthreads();
  put_adj<D, true>(r2, LD, sqs);  // S^T, from the S held in registers
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt) gtv[nt] = mma<D>(sV + trow * LD, LD, r2 + 16 * nt * LD, LD, z);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = trow + 4 * g + i;
    const float e = expf(bcum[kC - 1] - bcum[t]);
    float kh = 0.f, vg = 0.f;
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
      hk[nt][i] *= e;
      gk[nt][i] *= e;
      gtv[nt][i] *= e;
      const int col = 16 * nt + tl;
      kh = __builtin_fmaf(bf16_to_f32(sK[t * LD + col]), hk[nt][i], kh);
      vg = __builtin_fmaf(bf16_to_f32(sV[t * LD + col]), gk[nt][i], vg);
    }
    // dgamma prefix term: e^{b_e-b_t} beta_t (k_t^T Rb k_t + v_t^T S k_t), Rb = Rs/2 on k k^T
    const float a = group_sum<16>(0.5f * kh + vg);
    if (tl == 0) ta[t] = betas[t] * a;
  }
  // ---- the chunk's own reverse-causal terms ------------------------------------------
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt) {
    hk[nt] = mma<2 * kC>(sA3 + trow * L2, L2, sYX + 16 * nt * L2, L2, hk[nt]);
    gk[nt] -= mma<kC>(sA3 + trow * L2, L2, sDOT + 16 * nt * LC, LC, z);
    gtv[nt] = mma<kC>(sMvd + trow * LC, LC, sYX + 16 * nt * L2 + kC, L2, gtv[nt]);
  }
  // ---- outputs ------------------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = trow + 4 * g + i;
    const float bt = betas[t];
    float kh = 0.f, vg = 0.f;
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
      const int col = 16 * nt + tl;
      kh = __builtin_fmaf(bf16_to_f32(sK[t * LD + col]), hk[nt][i], kh);
      vg = __builtin_fmaf(bf16_to_f32(sV[t * LD + col]), gk[nt][i], vg);
    }
    const float dbeta = group_sum<16>(0.5f * kh + vg);
    if (t < Lc) {
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) {
        const int col = 16 * nt + tl;
        p.dk[(row0 + t) * D + col] = bt * (hk[nt][i] + gtv[nt][i]);
        p.dv[(row0 + t) * D + col] = bt * gk[nt][i];
      }
      if (tl == 0) p.dbeta[row0 + t] = dbeta;
    }
  }
  __syncthreads();
  // dgamma_t = (per-chunk + prefix + suffix + pair terms, every written token j < t) / gamma_t.
  // Each such term carries gamma_t (its decay runs from j past t), so the sum is
  // gamma_t <Hhat_t, H_{t-1}> + gamma_t <Ghat_t, G_{t-1}> formed directly: no
  // token's own term beta_t dbeta_t is added and taken out again, and the
  // division only rescales a sum that is already small when gamma_t is.
  if (wave == 0) {
    float A = ta[lane], R = trs[lane], Sf = tsuf[lane];
    float Cl = tcol[0][lane] + tcol[1][lane] + tcol[2][lane] + tcol[3][lane];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float a2 = __shfl_up(A, o, 64), r2v = __shfl_up(R, o, 64), c2 = __shfl_up(Cl, o, 64);
      const float s2 = __shfl_down(Sf, o, 64);
      if (lane >= o) {
        A += a2;
        R += r2v;
        Cl += c2;
      }
      if (lane + o < 64) Sf += s2;
    }
    // exclusive prefix sums (tokens u < t): the inclusive sums one token back
    // (every lane shuffles, then lane 0 takes zero)
    const float a1 = __shfl_up(A, 1, 64), r1v = __shfl_up(R, 1, 64), c1v = __shfl_up(Cl, 1, 64);
    const float Ae = lane > 0 ? a1 : 0.f;
    const float Re = lane > 0 ? r1v : 0.f;
    const float Ce = lane > 0 ? c1v : 0.f;
    // pairs j < t <= t': sum_{u<t} rowsum_u - sum_{u<t} colsum_u
    const float pairs = Re - Ce;
    const float c1 = expf(bcum[kC - 1]) *
                     (0.5f * (red[0][0] + red[0][1] + red[0][2] + red[0][3]) + red[1][0] + red[1][1] + red[1][2] + red[1][3]);
    if (lane < Lc) p.dgamma[row0 + lane] = (c1 + Ae + Sf + pairs) / p.gamma[row0 + lane];
  }
  (void)h;
}

// dlambda[h][i] = sum over the batch of the sequences' parts
__global__ __launch_bounds__(128) void bwd_lambda_kernel(BwdParams p, int D) {
  const int h = blockIdx.x;
  for (int i = threadIdx.x; i < D; i += 128) {
    float acc = 0.f;
    if (p.NC > 0)
      for (int b = 0; b < p.BH / p.H; ++b)
        for (int sg = 0; sg < p.NS; ++sg) acc += p.lam_part[((size_t)(b * p.H + h) * p.NS + sg) * D + i];
    p.dlam[h * D + i] = acc;
  }
}

// Partial sums of -y_t x_t^T over one split of the (b, t) rows of head h, for
// one 64 x 64 block (rows i of y, columns j of x).  y_t = nu_t * yn_t.  Each of
// the 256 threads owns a 4 x 4 patch; rows come through LDS in tiles of 64.
template <int D>
__global__ __launch_bounds__(256) void bwd_lamfull_part_kernel(BwdParams p) {
  // One workgroup forms the whole D x D partial sum of one head over one
  // split of its (b, t) rows, so every row of y and x is read once.  Rows are
  // staged 64 at a time in LDS; wave w owns the quadrant (w/2, w%2) and
  // contracts over the rows on fp32 MFMA (16x16x4): A = the staged y columns
  // of its row tiles, B = the staged x columns of its column tiles.  The next
  // 64 rows are loaded into registers while the current ones are multiplied.
  constexpr int LDP = D + 16;          // row stride (floats): 4 rows of 16 lanes hit distinct banks
  constexpr int QPR = D / 4;           // float4 quads per row
  constexpr int RPP = 256 / QPR;       // rows staged per pass of the workgroup
  constexpr int NP = 64 / RPP;         // passes per 64-row tile
  constexpr int TQ = D / 32;           // 16-wide tiles per side of a quadrant
  const int sp = blockIdx.x % kLamSplits;
  const int h = blockIdx.x / kLamSplits;
  const int B = p.BH / p.H;
  const long long R = (long long)B * p.T;  // rows (b, t) of head h
  const long long r_lo = R * sp / kLamSplits, r_hi = R * (sp + 1) / kLamSplits;
  __shared__ __attribute__((aligned(16))) float Ys[64 * LDP];
  __shared__ __attribute__((aligned(16))) float Xs[64 * LDP];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, tl = lane & 15, g = lane >> 4;
  const int q = tid % QPR, rr0 = tid / QPR;
  const int i0 = (wave >> 1) * (D / 2), j0 = (wave & 1) * (D / 2);

  f32x4 yv[NP], xv[NP];
  // rows r0 + o of the tile: (b, t) from one division per tile (uniform) and a
  // 32-bit division of the tile offset, not a 64-bit one per row.  The scale
  // nu is applied when the rows are stored to LDS, so the loads stay in flight
  // during the products of the current tile.
  float nv[NP];
  auto load_rows = [&](long long r0) {
    const long long b0 = r0 / p.T;
    const int t0 = (int)(r0 - b0 * p.T);
    const int rem = (int)min((long long)64, r_hi - r0);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int o = rr0 + RPP * u;
      yv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      xv[u] = yv[u];
      nv[u] = 0.f;
      if (o < rem) {
        const unsigned tt = (unsigned)(t0 + o), db = tt / (unsigned)p.T;
        const int t = (int)(tt - db * (unsigned)p.T);
        const size_t row = ((size_t)(b0 + db) * p.H + h) * p.T + t;
        yv[u] = *reinterpret_cast<const f32x4*>(p.yn + row * D + 4 * q);
        xv[u] = *reinterpret_cast<const f32x4*>(p.x + row * D + 4 * q);
        nv[u] = p.nu[row];
      }
    }
  };
  f32x4 acc[TQ][TQ];
#pragma unroll
  for (int a = 0; a < TQ; ++a)
#pragma unroll
    for (int c = 0; c < TQ; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (r_lo < r_hi) load_rows(r_lo);
  for (long long r0 = r_lo; r0 < r_hi; r0 += 64) {
    __syncthreads();  // the previous tile's reads are done
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      *reinterpret_cast<f32x4*>(Ys + (rr0 + RPP * u) * LDP + 4 * q) = yv[u] * nv[u];
      *reinterpret_cast<f32x4*>(Xs + (rr0 + RPP * u) * LDP + 4 * q) = xv[u];
    }
    __syncthreads();
    if (r0 + 64 < r_hi) load_rows(r0 + 64);
    // operands of step k4 + 1 are read from LDS while step k4's products issue
    float a[TQ], b[TQ];
#pragma unroll
    for (int it = 0; it < TQ; ++it) a[it] = Ys[g * LDP + i0 + 16 * it + tl];
#pragma unroll
    for (int jt = 0; jt < TQ; ++jt) b[jt] = Xs[g * LDP + j0 + 16 * jt + tl];
#pragma unroll
    for (int k4 = 0; k4 < 16; ++k4) {
      float an[TQ], bn[TQ];
      if (k4 < 15) {
        const int rk = (4 * (k4 + 1) + g) * LDP;
#pragma unroll
        for (int it = 0; it < TQ; ++it) an[it] = Ys[rk + i0 + 16 * it + tl];
#pragma unroll
        for (int jt = 0; jt < TQ; ++jt) bn[jt] = Xs[rk + j0 + 16 * jt + tl];
      }
#pragma unroll
      for (int it = 0; it < TQ; ++it)
#pragma unroll
        for (int jt = 0; jt < TQ; ++jt) acc[it][jt] = mfma_f32(a[it], b[jt], acc[it][jt]);
      if (k4 < 15) {
#pragma unroll
        for (int e = 0; e < TQ; ++e) {
          a[e] = an[e];
          b[e] = bn[e];
        }
      }
    }
  }
  float* out = p.lam_full_part + ((size_t)h * kLamSplits + sp) * D * D;
#pragma unroll
  for (int it = 0; it < TQ; ++it)
#pragma unroll
    for (int jt = 0; jt < TQ; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        out[(size_t)(i0 + 16 * it + 4 * g + e) * D + j0 + 16 * jt + tl] = -acc[it][jt][e];
}

// dLambda[h] = sum of the splits' partial sums
__global__ __launch_bounds__(256) void bwd_lamfull_sum_kernel(BwdParams p, int D) {
  const size_t n = (size_t)D * D;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;  // element of all heads
  if (e >= (size_t)p.H * n) return;
  const size_t h = e / n, ij = e % n;
  float acc = 0.f;
  for (int sp = 0; sp < kLamSplits; ++sp) acc += p.lam_full_part[(h * kLamSplits + sp) * n + ij];
  p.dlam[e] = acc;
}

template <int D>
hipError_t launch_bwd_d(int phase, const BwdParams& p, hipStream_t s) {
  const dim3 chunks((unsigned)(p.BH * p.NC));
  switch (phase) {
    case 0: hipLaunchKernelGGL((bwd_dx_kernel<D>), chunks, dim3(kThreads), 0, s, p); break;
    case 1: {
      // (sequence, stripe) units padded to whole groups of 8 sequences (one per XCD)
      if (bwd_scan_whole_state(p.BH, p.NS)) {
        // two workgroups per sequence, padded to whole groups of 8 sequences (one per XCD)
        const unsigned wgs = (unsigned)((p.BH + 7) / 8 * 8 * 2);
        hipLaunchKernelGGL((bwd_scan_full_kernel<D>), dim3(wgs), dim3(kFullThreads), 0, s, p);
        break;
      }
      const unsigned units = (unsigned)((p.BH + 7) / 8 * 8 * (D / 32));
      if (p.NS > 1) {
        hipLaunchKernelGGL((bwd_scan_kernel<D, true>), dim3(units * (unsigned)(p.NS - 1)), dim3(kThreads), 0, s, p);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        const long long n = (long long)p.BH * 2 * D * D;
        hipLaunchKernelGGL(bwd_carry_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, D);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      }
      hipLaunchKernelGGL((bwd_scan_kernel<D, false>), dim3(units * (unsigned)p.NS), dim3(kThreads), 0, s, p);
      break;
    }
    case 2:
      if (p.NC > 0) {
        hipLaunchKernelGGL((bwd_grad_kernel<D>), chunks, dim3(kThreads), 0, s, p);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      }
      if (p.lam_full) {
        hipLaunchKernelGGL((bwd_lamfull_part_kernel<D>), dim3((unsigned)(p.H * kLamSplits)), dim3(256), 0,
                           s, p);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        const size_t n = (size_t)p.H * D * D;
        hipLaunchKernelGGL(bwd_lamfull_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, D);
      } else {
        hipLaunchKernelGGL(bwd_lambda_kernel, dim3((unsigned)p.H), dim3(128), 0, s, p, D);
      }
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(int phase, int D, const BwdParams& p, hipStream_t s) {
  if (D == 128) return launch_bwd_d<128>(phase, p, s);
  if (D == 64) return launch_bwd_d<64>(phase, p, s);
  return hipErrorInvalidValue;
}

}  // namespace mesa
