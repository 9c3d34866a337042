// One token row of the query/key preprocessing (MesaNet page, "architecture":
// queries and keys are normalised and convolved with a small window before the
// layer): the causal depthwise convolution of 8 consecutive channels and the
// row's L2 normalisation,
//     y_t[j] = sum_{i < W} w[h][j][i] x_{t-i}[j],   out_t = y_t / max(||y_t||, eps).
// Every kernel that forms processed rows -- the standalone preprocessing
// kernel and the scan and CG kernels of the fused forward -- uses these
// helpers with a row's D/8 lanes side by side in one wave and group_sum over
// them, so all of them produce the same bf16 values.
#pragma once

#include <type_traits>

#include "mesa_common.h"

namespace mesa {

// This lane's taps w[h][c0 + e][i] (e < 8, i < W), from [H, D, W] fp32.
template <int W>
__device__ __forceinline__ void prep_taps8(const float* taps, int h, int D, int c0, float (&w)[8][W]) {
  const float* wp = taps + ((size_t)h * D + c0) * W;
#pragma unroll
  for (int i4 = 0; i4 < 2 * W; ++i4) {
    const f32x4 t = reinterpret_cast<const f32x4*>(wp)[i4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[(4 * i4 + u) / W][(4 * i4 + u) % W] = t[u];
  }
}

// Convolved channels y[e] of one token from its raw rows x[m] = x_{t-(W-1)+m}
// (zero before a sequence without history), tap 0 first; returns this lane's
// part of ||y||^2 (the caller sums it over the row's lanes with group_sum).
template <int W>
__device__ __forceinline__ float prep_conv8(const float (&w)[8][W], const float (&x)[W][8], float (&y)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < W; ++i) acc = __builtin_fmaf(w[e][i], x[W - 1 - i][e], acc);
    y[e] = acc;
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(y[e], y[e], ss);
  return ss;
}

// 1 / max(||y||, eps) from the row's summed squares ss, as
// min(1/sqrt(ss), 1/eps) with the hardware reciprocal square root (1 ulp).
// ss is raised to the smallest normal float first: below it ||y|| < 2^-63,
// which is below every eps the entry points accept, so the result is 1/eps
// either way, and the reciprocal square root never sees a denormal.
__device__ __forceinline__ float prep_scale(float ss, float inv_eps) {
  return fminf(__builtin_amdgcn_rsqf(fmaxf(ss, 0x1p-126f)), inv_eps);
}

// The sum over a row's N = D/8 channel-group partials p[0..N) in the order
// group_sum<N> adds them across lanes (a balanced pairwise tree: each DPP
// level adds two equal-sized subtrees, and fp32 addition commutes exactly).
template <int N>
__device__ __forceinline__ float prep_tree_sum(const float* p) {
  if constexpr (N == 1) {
    return p[0];
  } else {
    return prep_tree_sum<N / 2>(p) + prep_tree_sum<N / 2>(p + N / 2);
  }
}

// 8 raw bf16 channels as fp32.
__device__ __forceinline__ void prep_unpack8(const u16x8& v, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(v[e]);
}

// The fused kernels take the window W (1..4) at run time, keep the last
// kPrepMaxW raw rows, and branch once on W to code built for that window:
// prep_conv8_pad<W> issues exactly the fma sequence of prep_conv8<W> (taps
// i < W, tap 0 first), so the values are the same.
constexpr int kPrepMaxW = 4;

__device__ __forceinline__ void prep_taps8_w(const float* taps, int h, int D, int c0, int W,
                                             float (&w)[8][kPrepMaxW]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int i = 0; i < kPrepMaxW; ++i) w[e][i] = i < W ? taps[((size_t)h * D + c0 + e) * W + i] : 0.f;
}

// prep_conv8<W> on the padded layout x[m] = x_{t-(kPrepMaxW-1)+m}, taps
// w[e][i] (i < kPrepMaxW, used for i < W).
template <int W>
__device__ __forceinline__ float prep_conv8_pad(const float (&w)[8][kPrepMaxW], const float (&x)[kPrepMaxW][8],
                                                float (&y)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < W; ++i) acc = __builtin_fmaf(w[e][i], x[kPrepMaxW - 1 - i][e], acc);
    y[e] = acc;
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(y[e], y[e], ss);
  return ss;
}

// Calls fn(std::integral_constant<int, W>) for the run-time window W (1..4).
template <typename F>
__device__ __forceinline__ void prep_with_window(int W, F&& fn) {
  switch (W) {
    case 1: fn(std::integral_constant<int, 1>{}); break;
    case 2: fn(std::integral_constant<int, 2>{}); break;
    case 3: fn(std::integral_constant<int, 3>{}); break;
    default: fn(std::integral_constant<int, 4>{}); break;
  }
}

// Raw channels c0..c0+7 of token r (any r < T) for a window of W: rows r >= 0
// from `raw`, rows -(W-1) <= r < 0 from `hist` when given.  Every other row
// (before the history, or before a sequence without one) is zero: the load is
// unconditional (it reads row 0 of the sequence) and prep_zero_row clears it
// where it is used, so that nothing waits for the load at the load.
__device__ __forceinline__ u16x8 prep_load8_w(const uint16_t* raw, const uint16_t* hist, int bh, int T, int D, int W,
                                              int r, int c0) {
  const bool from_hist = r < 0 && hist && r >= -(W - 1);
  const uint16_t* src = from_hist ? hist + ((size_t)bh * (W - 1) + (W - 1 + r)) * D + c0
                                  : raw + ((size_t)bh * T + min(max(r, 0), T - 1)) * D + c0;
  return *reinterpret_cast<const u16x8*>(src);
}

// Row r as the window sees it: zero before the history (or before a sequence
// without one), else the loaded bits.
__device__ __forceinline__ u16x8 prep_zero_row(const u16x8& v, const void* hist, int W, int r) {
  const bool zero = r < 0 && !(hist && r >= -(W - 1));
  return zero ? u16x8{0, 0, 0, 0, 0, 0, 0, 0} : v;
}

// One wave forms the processed rows 0..C-1 of the chunk of tokens s..s+C-1 of
// sequence bh (head h) into dst[j * stride + c] as bf16.  A row's D/8 lanes
// sit side by side, so 64/(D/8) rows are formed at once and each lane group
// walks C/(64/(D/8)) consecutive rows, from its raw rows (the window's
// earlier rows included) loaded in one batch by load(), so that the caller
// can issue the loads early; form() then needs no memory but the taps.  Rows
// past the chunk's Lc tokens repeat its last raw row: finite values that the
// callers ignore.
template <int D, int C>
struct PrepChunk {
  static constexpr int LPR = D / 8, NG = 64 / LPR, RPG = C / NG, NR = RPG + kPrepMaxW - 1;
  static_assert(NG * RPG == C, "whole rows per lane group");
  u16x8 rr[NR];
  const void* hist_;
  int s_;

  __device__ __forceinline__ void load(const uint16_t* raw, const uint16_t* hist, int bh, int T, int W, int s,
                                       int Lc, int lane) {
    const int c0 = 8 * (lane % LPR), j0 = (lane / LPR) * RPG;
    hist_ = hist;
    s_ = s;
#pragma unroll
    for (int m = 0; m < NR; ++m)
      rr[m] = prep_load8_w(raw, hist, bh, T, D, W, min(s + j0 - (kPrepMaxW - 1) + m, s + Lc - 1), c0);
  }

  __device__ __forceinline__ void form(const float* taps, int h, int W, float inv_eps, __bf16* dst, int stride,
                                       int lane) const {
    const int c0 = 8 * (lane % LPR), j0 = (lane / LPR) * RPG;
    u16x8 zr[NR];
#pragma unroll
    for (int m = 0; m < NR; ++m) zr[m] = prep_zero_row(rr[m], hist_, W, s_ + j0 - (kPrepMaxW - 1) + m);
    float w[8][kPrepMaxW];
    prep_taps8_w(taps, h, D, c0, W, w);
    prep_with_window(W, [&](auto wc) {
      constexpr int WW = decltype(wc)::value;
#pragma unroll
      for (int r = 0; r < RPG; ++r) {
        float x8[kPrepMaxW][8], y[8];
#pragma unroll
        for (int m = kPrepMaxW - WW; m < kPrepMaxW; ++m) prep_unpack8(zr[r + m], x8[m]);
        const float sc = prep_scale(group_sum<LPR>(prep_conv8_pad<WW>(w, x8, y)), inv_eps);
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (__bf16)(y[e] * sc);
        *reinterpret_cast<bf16x8*>(dst + (size_t)(j0 + r) * stride + c0) = o;
      }
    });
  }
};

}  // namespace mesa
