// Internal launch interface between the C ABI (mesa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mesa {

// Chunk-boundary state scan (one pass over the chunks of every (b, h)).
struct ScanParams {
  const void* k;         // [BH, T, D] bf16 or fp32
  const void* v;         // [BH, T, D]
  const float* gamma;    // [BH, T]
  const float* beta;     // [BH, T]
  const float* h0;       // [BH, D, D] or null
  const float* g0;       // [BH, D, D] or null
  float* h_final;        // [BH, D, D] or null
  float* g_final;        // [BH, D, D] or null
  void* hb;              // [BH, NC, D*D] boundary snapshots of H (layout: see scan kernel)
  void* gb;              // [BH, NC, D*D] boundary snapshots of G
  int BH, T, NC;
  // segmented walk (long sequences with few (b, h)): NS segments of SEG chunks
  int SEG, NS;
  float* seg_state;      // [BH, 2, NS-1, D*D]: segment totals, then carry-in states
  float* seg_decay;      // [BH, NS-1]: product of gamma over each segment
  // fused preprocessing (bf16, chunk 64): k holds raw keys, convolved with the
  // taps wk [H, D, W] and L2-normalised (eps) as they are staged; k_hist
  // [BH, W-1, D] raw keys before t = 0, or null (zeros)
  int prep, W, H;
  const float* wk;
  const void* k_hist;
  float inv_eps;         // 1 / eps
};

// Segments per sequence for the state scan.  Whole-state workgroups (one per
// CU) fill the GPU with one walk once 2*BH >= 256.  With fewer (b, h) and a
// long sequence (>= 128 chunks) the whole-state walk is split into segments,
// about 256 workgroups in all with at least 8 chunks each; shorter sequences
// walk once in 16-row stripes (segmenting stripes does not pay: every stripe
// stages the whole chunk).
inline int scan_segments(long long BH, int NC, int D) {
  (void)D;
  if (2 * BH >= 256 || NC < 128) return 1;
  long long ns = (256 + 2 * BH - 1) / (2 * BH);
  if (ns > NC / 8) ns = NC / 8;
  if (ns < 2) return 1;
  const int seg = (int)((NC + ns - 1) / ns);
  return (NC + seg - 1) / seg;
}
// whole-state workgroups (else 16-row stripes)
inline bool scan_whole_state(long long BH, int NC, int D) { return 2 * BH >= 256 || scan_segments(BH, NC, D) > 1; }
inline int scan_segment_chunks(int NC, int NS) { return (NC + NS - 1) / NS; }
inline size_t scan_segment_bytes(long long BH, int NC, int D) {
  const int ns = scan_segments(BH, NC, D);
  if (ns <= 1) return 0;
  const size_t st = (size_t)BH * 2 * (ns - 1) * D * D * 4;
  const size_t dec = ((size_t)BH * (ns - 1) * 4 + 255) / 256 * 256;
  return st + dec;
}

// Chunked CG solve + output.
struct CgParams {
  const void* q;         // [BH, T, D]
  const void* k;
  const void* v;
  const float* gamma;    // [BH, T]
  const float* beta;
  const float* lam;      // [H, D] diagonal, or [H, D, D] with lam_full
  const void* hb;        // snapshots written by the scan
  const void* gb;
  float* o;              // [BH, T, D]; null on the bf16 path: solutions only, no read-out
  int32_t* steps;        // [BH, T] or null
  float* x_out;          // [BH, T, D] or null
  int32_t* unscaled;     // [BH, NC] bf16 path: chunks left to the unscaled kernel
  int BH, H, T, NC, max_steps;
  float tol2;            // tol*tol, or -1 for the fixed-step mode
  int lam_full;          // lam is a full symmetric matrix per head (bf16 path, chunk 64, D 64 or 128)
  int warm;              // bf16 path, diagonal Lambda: token t's CG starts from token t-16's
                         // solution when both lie in one chunk (tiles 1.. of a chunk)
  // fused preprocessing (bf16, diagonal Lambda, chunk 64, D 64 or 128): q and k
  // hold raw vectors, convolved with the taps wq / wk [H, D, W] and
  // L2-normalised (eps) as they are loaded; q_hist / k_hist [BH, W-1, D] raw
  // vectors before t = 0, or null (zeros)
  int prep, W;
  const float* wq;
  const float* wk;
  const void* q_hist;
  const void* k_hist;
  float inv_eps;         // 1 / eps
};

// Largest total decay -sum(log gamma) of a chunk that the scaled bf16 CG kernel
// handles: e^40 keeps its decay-scaled weights far inside the fp32 range.
constexpr float kMaxScaledDecay = 40.f;

struct DecodeParams {
  const void* q;         // [P, D]  (P = N*H pairs)
  const void* k;
  const void* v;
  const float* gamma;    // [P]
  const float* beta;
  const float* lam;      // [H, D] diagonal, or [H, D, D] with lam_full
  float* h;              // [P, D, D] in/out
  float* g;              // [P, D, D] in/out
  float* o;              // [P, D]
  int32_t* steps;        // [P] or null
  float* x_out;          // [P, D] or null
  const float* x0;       // [P, D] CG start (warm variant only; may alias x_out)
  int P, H, max_steps;
  float tol2;
  int lam_full;          // lam is a full symmetric matrix per head
};

// Query/key preprocessing: index 0 = queries, 1 = keys.
struct PrepParams {
  const void* x[2];        // raw [BH, T, D]
  const float* w[2];       // taps [H, D, W]
  const void* hist_in[2];  // [BH, W-1, D] or null (zeros)
  void* out[2];            // [BH, T, D]
  void* hist_out[2];       // [BH, W-1, D] or null
  int BH, H, T, W;
  float inv_eps;           // 1 / eps
};

// Backward pass (bf16 inputs, chunk 64).
struct BwdParams {
  const void* k;            // [BH, T, D] bf16
  const void* v;
  const float* gamma;       // [BH, T]
  const float* beta;
  const void* hb;           // forward boundary snapshots (bf16 fragment order)
  const void* gb;
  const float* x;           // forward solutions [BH, T, D]
  const float* d_o;         // dL/do
  const float* d_hfinal;    // [BH, D, D] or null
  const float* d_gfinal;
  void* rhs;                // adjoint right-hand sides dx/||dx|| [BH, T, D] bf16
  float* nu;                // ||dx|| [BH, T]
  const float* yn;          // adjoint CG solutions for rhs [BH, T, D]
  uint16_t* snap_r;         // per chunk: Hhat + Hhat^T and Ghat at its end [BH*NC, D, D] bf16
  uint16_t* snap_s;
  float* dq;                // [BH, T, D]
  float* dk;
  float* dv;
  float* dbeta;             // [BH, T]
  float* dgamma;
  float* lam_part;          // [BH, NS, D]: -sum_t y_t * x_t per sequence segment
  float* dlam;              // [H, D]
  float* dh0;               // [BH, D, D] or null
  float* dg0;
  // adjoint scan of a long sequence in NS segments of SEG chunks (NS = 1: one walk)
  float* seg_state;         // [BH, 2, NS-1, D*D]: segment totals, then carry-in states
  float* seg_decay;         // [BH, NS-1]: total decay of segments 1..NS-1
  int BH, H, T, NC, NS, SEG;
  // a full Lambda: dlam is [H, D, D], summed from kLamSplits partial sums per head
  int lam_full;
  float* lam_full_part;     // [H, kLamSplits, D, D]
};

// Row splits of the full-Lambda gradient -sum_{b,t} y_t x_t^T per head.
constexpr int kLamSplits = 32;

// Segments of the adjoint scan: a sequence is split when there are too few
// (sequence, 32-row stripe) units to fill the chip (two resident workgroups per CU)
// and the sequence is long.
inline int bwd_scan_segments(long long BH, int NC, int D) {
  const long long units = BH * (D / 32);
  if (units >= 256 || NC < 128) return 1;
  long long ns = (512 + units - 1) / units;
  if (ns > NC / 16) ns = NC / 16;
  if (ns < 2) return 1;
  const int seg = (int)((NC + ns - 1) / ns);
  return (NC + seg - 1) / seg;
}

// The adjoint scan walks whole states (two workgroups per sequence, one per CU)
// once there are enough sequences to fill the chip, else 32-row stripes.
inline bool bwd_scan_whole_state(long long BH, int NS) { return 2 * BH >= 256 && NS == 1; }

// Each returns hipSuccess or the launch error.
hipError_t launch_scan(bool bf16, int D, int C, const ScanParams& p, hipStream_t s);
hipError_t launch_cg(bool bf16, int D, int C, const CgParams& p, hipStream_t s);
hipError_t launch_cg_bf16(int D, int C, const CgParams& p, hipStream_t s);
hipError_t launch_cg_bf16_unscaled(int D, int C, const CgParams& p, hipStream_t s);
// packed_h: DecodeParams::h in the blocked upper-triangular layout;
// warm: CG starts from DecodeParams::x0
hipError_t launch_decode(bool bf16, int D, bool packed_h, bool warm, const DecodeParams& p, hipStream_t s);
// phase 0: adjoint right-hand sides; 1: adjoint scan; 2: per-token gradients and dlambda
hipError_t launch_bwd(int phase, int D, const BwdParams& p, hipStream_t s);
hipError_t launch_qk_prep(bool bf16, int D, const PrepParams& p, hipStream_t s);
hipError_t launch_sym_pack(int D, int count, const float* full, float* packed, hipStream_t s);
hipError_t launch_sym_unpack(int D, int count, const float* packed, float* full, hipStream_t s);
size_t sym_state_floats(int D);

// Bytes of one (b, h, chunk) boundary snapshot of H (or of G).
inline size_t snapshot_bytes(bool bf16, int D) { return (size_t)D * D * (bf16 ? 2 : 4); }

// Bytes of the per-chunk form flags of the bf16 path (whole 256-byte blocks).
inline size_t flag_bytes(size_t chunks) { return (chunks * 4 + 255) / 256 * 256; }

}  // namespace mesa
