// Packed-symmetric storage of the key-covariance state H for the decode step.
//
// MesaNet page, technical summary, "Mesa layer" section: H_t = gamma_t H_{t-1}
// + beta_t k_t k_t^T is symmetric, so its upper triangle carries all of it; the
// decode step is bound by streaming the states through HBM, and storing H
// packed cuts the bytes it moves.
//
// Layout ("blocked upper triangle"): the d/16 x d/16 grid of 16x16 blocks,
// upper triangle including the diagonal, in row-major block order (0,0),
// (0,1), ..., (0,nb-1), (1,1), ...; every block is 16x16 fp32 row-major (1 KB),
// block (bi, bj) holding H[16 bi + r][16 bj + c].  Diagonal blocks are stored
// whole.  This file converts between the full and the packed layout; the
// decode step on packed states is the decode kernel's SYMH variant
// (mesa_decode.hip).
#include "mesa_common.h"
#include "mesa_kernels.h"

namespace mesa {

namespace {

template <int D>
struct SymShape {
  static constexpr int NB = D / 16;                      // blocks per side
  static constexpr int NBLK = NB * (NB + 1) / 2;         // stored blocks
};

// row-major index of block (bi, bj), bi <= bj, in the upper triangle of an nb x nb grid
__device__ __forceinline__ int sym_block(int nb, int bi, int bj) { return bi * nb - bi * (bi - 1) / 2 + (bj - bi); }

__device__ __forceinline__ void sym_block_rc(int nb, int b, int& bi, int& bj) {
  bi = 0;
  while (b >= nb - bi) {
    b -= nb - bi;
    ++bi;
  }
  bj = bi + b;
}

// full [count][D][D] -> packed: one workgroup per stored block
template <int D>
__global__ __launch_bounds__(256) void sym_pack_kernel(const float* full, float* packed, int count) {
  constexpr int NB = SymShape<D>::NB, NBLK = SymShape<D>::NBLK;
  const long long blk = blockIdx.x;
  const long long s = blk / NBLK;
  if (s >= count) return;
  int bi, bj;
  sym_block_rc(NB, (int)(blk % NBLK), bi, bj);
  const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
  packed[blk * 256 + threadIdx.x] = full[(size_t)s * D * D + (size_t)(16 * bi + r) * D + 16 * bj + c];
}

// packed -> full, the lower blocks mirrored from the upper ones
template <int D>
__global__ __launch_bounds__(256) void sym_unpack_kernel(const float* packed, float* full, int count) {
  constexpr int NB = SymShape<D>::NB, NBLK = SymShape<D>::NBLK;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)count * D * D) return;
  const long long s = idx / (D * D);
  const int i = (int)(idx % (D * D)) / D, j = (int)(idx % D);
  const int bi = i >> 4, bj = j >> 4;
  const float v = bi <= bj ? packed[(s * NBLK + sym_block(NB, bi, bj)) * 256 + (i & 15) * 16 + (j & 15)]
                           : packed[(s * NBLK + sym_block(NB, bj, bi)) * 256 + (j & 15) * 16 + (i & 15)];
  full[idx] = v;
}

}  // namespace

size_t sym_state_floats(int D) {
  const size_t nb = (size_t)D / 16;
  return nb * (nb + 1) / 2 * 256;
}

hipError_t launch_sym_pack(int D, int count, const float* full, float* packed, hipStream_t s) {
  if (D == 128) {
    hipLaunchKernelGGL((sym_pack_kernel<128>), dim3((unsigned)((long long)count * SymShape<128>::NBLK)), dim3(256), 0, s,
                       full, packed, count);
  } else if (D == 64) {
    hipLaunchKernelGGL((sym_pack_kernel<64>), dim3((unsigned)((long long)count * SymShape<64>::NBLK)), dim3(256), 0, s,
                       full, packed, count);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sym_unpack(int D, int count, const float* packed, float* full, hipStream_t s) {
  const long long n = (long long)count * D * D;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (D == 128) hipLaunchKernelGGL((sym_unpack_kernel<128>), grid, dim3(256), 0, s, packed, full, count);
  else if (D == 64) hipLaunchKernelGGL((sym_unpack_kernel<64>), grid, dim3(256), 0, s, packed, full, count);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mesa
