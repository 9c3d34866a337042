// Query/key preprocessing ahead of the Mesa layer: a causal depthwise
// convolution along time, then L2 normalisation of every token vector.
//
// MesaNet page, "architecture" section: queries and keys are normalised and
// convolved with a small window before the layer.  Taken as
//     y_t[j] = sum_{i < W} w[h][j][i] * x_{t-i}[j],    out_t = y_t / max(||y_t||_2, eps)
// (convolution first, so the layer receives unit-norm vectors).  The W-1 raw
// vectors before t = 0 come from a history buffer (a continued sequence or a
// decode step) or are zero.
//
// The kernel is bound by HBM: each raw vector is read once and each output
// written once.  A token row of D channels is spread over LPR = D/8 lanes
// holding 8 consecutive channels each (one 16-byte bf16 or two 16-byte fp32
// loads), so a wave instruction covers 64/LPR rows.  Every lane group walks S
// consecutive tokens of one (b, h) and also loads the W-1 rows before its
// range (the previous group's last rows, so those reads mostly hit in cache);
// all S+W-1 rows are loaded into registers before the first is used.  The
// squared norm is summed over the LPR lanes of a row with DPP moves.
#include "mesa_common.h"
#include "mesa_kernels.h"
#include "mesa_prep_rows.h"

namespace mesa {

namespace {

constexpr int kPrepThreads = 256;

template <bool BF16>
struct Row8;  // 8 consecutive channels of one token, as stored
template <>
struct Row8<true> {
  u16x8 v;
  __device__ float at(int e) const { return bf16_to_f32(v[e]); }
};
template <>
struct Row8<false> {
  f32x4 a, b;
  __device__ float at(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

template <bool BF16>
__device__ __forceinline__ Row8<BF16> load_row8(const void* base, size_t elem) {
  Row8<BF16> r;
  if constexpr (BF16) {
    r.v = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(base) + elem);
  } else {
    const f32x4* ptr = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
    r.a = ptr[0];
    r.b = ptr[1];
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ void store_row8(void* base, size_t elem, const float (&y)[8]) {
  if constexpr (BF16) {
    u16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = __builtin_bit_cast(uint16_t, f32_to_bf16(y[e]));
    *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(base) + elem) = o;
  } else {
    f32x4* ptr = reinterpret_cast<f32x4*>(static_cast<float*>(base) + elem);
    ptr[0] = f32x4{y[0], y[1], y[2], y[3]};
    ptr[1] = f32x4{y[4], y[5], y[6], y[7]};
  }
}

template <bool BF16, int D>
struct PrepShape {
  static constexpr int LPR = D / 8;                 // lanes per token row
  static constexpr int GPW = 64 / LPR;              // rows side by side in a wave
  static constexpr int S = 8;                       // tokens per lane group
  static constexpr int NG = (kPrepThreads / 64) * GPW;
  static constexpr int TILE = NG * S;               // tokens per workgroup
};

template <bool BF16, int D, int W>
__global__ __launch_bounds__(kPrepThreads) void qk_prep_kernel(PrepParams p) {
  using Sh = PrepShape<BF16, D>;
  constexpr int LPR = Sh::LPR, S = Sh::S, NR = S + W - 1;
  const int which = blockIdx.z;  // 0: queries, 1: keys
  const int bh = blockIdx.y;
  const int h = bh % p.H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = 8 * (lane % LPR);
  const int t0 = blockIdx.x * Sh::TILE + (wave * Sh::GPW + lane / LPR) * S;
  const void* x = p.x[which];
  const void* hist = p.hist_in[which];

  // rows t0-W+1 .. t0+S-1: rows past the end are clamped (never stored),
  // rows before 0 come from the history or are zero
  Row8<BF16> rows[NR];
  bool zero[NR];
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    const int r = t0 - (W - 1) + m;
    const bool before = r < 0;
    const void* src = before && hist ? hist : x;
    const size_t elem = before && hist ? ((size_t)bh * (W - 1) + (W - 1 + r)) * D + c0
                                       : ((size_t)bh * p.T + min(max(r, 0), p.T - 1)) * D + c0;
    rows[m] = load_row8<BF16>(src, elem);
    zero[m] = before && !hist;
  }
  // this lane's taps: 8 channels x W, contiguous
  float w[8][W];
  prep_taps8<W>(p.w[which], h, D, c0, w);

  void* out = p.out[which];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    float x8[W][8], y[8];
#pragma unroll
    for (int m = 0; m < W; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) x8[m][e] = zero[s + m] ? 0.f : rows[s + m].at(e);
    const float ss = group_sum<LPR>(prep_conv8<W>(w, x8, y));
    const float scale = prep_scale(ss, p.inv_eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] *= scale;
    const int t = t0 + s;
    if (t < p.T) store_row8<BF16>(out, ((size_t)bh * p.T + t) * D + c0, y);
  }
}

// The next call's history: the last W-1 raw vectors of [history, sequence].
template <bool BF16>
__global__ __launch_bounds__(256) void qk_prep_history_kernel(PrepParams p, int D) {
  const int W1 = p.W - 1;
  const long long n = (long long)p.BH * W1 * D;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const int which = blockIdx.y;
  if (idx >= n || !p.hist_out[which]) return;
  const int j = (int)(idx % D);
  const int i = (int)((idx / D) % W1);
  const long long bh = idx / ((long long)D * W1);
  const int r = p.T - W1 + i;
  float v = 0.f;
  if (r >= 0) v = load1<BF16>(p.x[which], ((size_t)bh * p.T + r) * D + j);
  else if (p.hist_in[which]) v = load1<BF16>(p.hist_in[which], ((size_t)bh * W1 + W1 + r) * D + j);
  if constexpr (BF16) {
    static_cast<uint16_t*>(p.hist_out[which])[idx] = __builtin_bit_cast(uint16_t, f32_to_bf16(v));
  } else {
    static_cast<float*>(p.hist_out[which])[idx] = v;
  }
}

template <bool BF16, int D, int W>
hipError_t launch_prep_t(const PrepParams& p, hipStream_t s) {
  using Sh = PrepShape<BF16, D>;
  const dim3 grid((unsigned)((p.T + Sh::TILE - 1) / Sh::TILE), (unsigned)p.BH, 2);
  hipLaunchKernelGGL((qk_prep_kernel<BF16, D, W>), grid, dim3(kPrepThreads), 0, s, p);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_prep_w(const PrepParams& p, hipStream_t s) {
  switch (p.W) {
    case 1: return launch_prep_t<BF16, D, 1>(p, s);
    case 2: return launch_prep_t<BF16, D, 2>(p, s);
    case 3: return launch_prep_t<BF16, D, 3>(p, s);
    case 4: return launch_prep_t<BF16, D, 4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16>
hipError_t launch_prep_d(int D, const PrepParams& p, hipStream_t s) {
  switch (D) {
    case 16: return launch_prep_w<BF16, 16>(p, s);
    case 64: return launch_prep_w<BF16, 64>(p, s);
    case 128: return launch_prep_w<BF16, 128>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_qk_prep(bool bf16, int D, const PrepParams& p, hipStream_t s) {
  // without outputs only the next call's histories are formed (the fused forward)
  if (p.T > 0 && p.out[0] && p.out[1]) {
    const hipError_t e = bf16 ? launch_prep_d<true>(D, p, s) : launch_prep_d<false>(D, p, s);
    if (e != hipSuccess) return e;
  }
  if (p.W > 1 && (p.hist_out[0] || p.hist_out[1])) {
    const long long n = (long long)p.BH * (p.W - 1) * D;
    const dim3 grid((unsigned)((n + 255) / 256), 2);
    if (bf16) hipLaunchKernelGGL((qk_prep_history_kernel<true>), grid, dim3(256), 0, s, p, D);
    else hipLaunchKernelGGL((qk_prep_history_kernel<false>), grid, dim3(256), 0, s, p, D);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mesa
