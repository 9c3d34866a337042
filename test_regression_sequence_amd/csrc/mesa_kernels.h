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
};

// Chunked CG solve + output.
struct CgParams {
  const void* q;         // [BH, T, D]
  const void* k;
  const void* v;
  const float* gamma;    // [BH, T]
  const float* beta;
  const float* lam;      // [H, D]
  const void* hb;        // snapshots written by the scan
  const void* gb;
  float* o;              // [BH, T, D]
  int32_t* steps;        // [BH, T] or null
  float* x_out;          // [BH, T, D] or null
  int32_t* unscaled;     // [BH, NC] bf16 path: chunks left to the unscaled kernel
  int BH, H, T, NC, max_steps;
  float tol2;            // tol*tol, or -1 for the fixed-step mode
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
  const float* lam;      // [H, D]
  float* h;              // [P, D, D] in/out
  float* g;              // [P, D, D] in/out
  float* o;              // [P, D]
  int32_t* steps;        // [P] or null
  float* x_out;          // [P, D] or null
  int P, H, max_steps;
  float tol2;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_scan(bool bf16, int D, int C, const ScanParams& p, hipStream_t s);
hipError_t launch_cg(bool bf16, int D, int C, const CgParams& p, hipStream_t s);
hipError_t launch_cg_bf16(int D, int C, const CgParams& p, hipStream_t s);
hipError_t launch_cg_bf16_unscaled(int D, int C, const CgParams& p, hipStream_t s);
hipError_t launch_decode(bool bf16, int D, const DecodeParams& p, hipStream_t s);

// Bytes of one (b, h, chunk) boundary snapshot of H (or of G).
inline size_t snapshot_bytes(bool bf16, int D) { return (size_t)D * D * (bf16 ? 2 : 4); }

// Bytes of the per-chunk form flags of the bf16 path (whole 256-byte blocks).
inline size_t flag_bytes(size_t chunks) { return (chunks * 4 + 255) / 256 * 256; }

}  // namespace mesa
