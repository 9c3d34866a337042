// C ABI of libmesa: argument validation, workspace carving, kernel launches.
// Every check runs before the first launch, so a failing call writes nothing.
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/mesa.h"
#include "mesa_kernels.h"

namespace {

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool supported_dim(mesa_dtype dt, int d) {
  if (dt == MESA_F32) return d == 16 || d == 32 || d == 64 || d == 128;
  return d == 32 || d == 64 || d == 128;
}

mesa_status check_desc(const mesa_fwd_desc* d) {
  if (!d) return MESA_ERR_INVALID_ARG;
  if (d->B < 1 || d->H < 1 || d->T < 0 || d->dk < 1 || d->dv < 1 || d->chunk < 1 || d->max_steps < 0)
    return MESA_ERR_INVALID_ARG;
  if (d->in_dtype != MESA_F32 && d->in_dtype != MESA_BF16) return MESA_ERR_INVALID_ARG;
  if (std::isnan(d->tol)) return MESA_ERR_INVALID_ARG;
  if (d->dk != d->dv || !supported_dim(d->in_dtype, d->dk)) return MESA_ERR_UNSUPPORTED;
  if (d->chunk != 16 && d->chunk != 32 && d->chunk != 64) return MESA_ERR_UNSUPPORTED;
  // grid and index ranges used by the kernels
  const long long bh = (long long)d->B * d->H;
  const long long nc = (d->T + d->chunk - 1) / d->chunk;
  if (bh > (1LL << 24) || bh * nc > (1LL << 31) - 1 || bh * d->T * (long long)d->dk > (1LL << 40))
    return MESA_ERR_UNSUPPORTED;
  return MESA_OK;
}

// The preprocessing's eps: finite and at least 2^-63 (below it the
// normalisation would need the norm of a vector whose squared norm is a
// denormal float).
bool eps_ok(float eps) { return eps >= 0x1p-63f && !std::isinf(eps); }

}  // namespace

extern "C" {

int32_t mesa_abi_version(void) { return MESA_ABI_VERSION; }

const char* mesa_status_string(mesa_status s) {
  switch (s) {
    case MESA_OK: return "ok";
    case MESA_ERR_INVALID_ARG: return "invalid argument";
    case MESA_ERR_UNSUPPORTED: return "unsupported size or configuration";
    case MESA_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case MESA_ERR_WORKSPACE: return "workspace missing or too small";
    case MESA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t mesa_fwd_workspace_bytes(const mesa_fwd_desc* d) {
  if (check_desc(d) != MESA_OK || d->T == 0) return 0;
  const size_t nc = (size_t)(d->T + d->chunk - 1) / d->chunk;
  const size_t bh = (size_t)d->B * d->H;
  const bool bf16 = d->in_dtype == MESA_BF16;
  return 2 * bh * nc * mesa::snapshot_bytes(bf16, d->dk) + (bf16 ? mesa::flag_bytes(bh * nc) : 0) +
         mesa::scan_segment_bytes((long long)bh, (int)nc, d->dk);
}

}  // extern "C"

namespace {

enum Phase { kScan = 1, kSolve = 2 };

// every check of a forward call except the workspace's size
mesa_status fwd_validate(int phases, const mesa_fwd_desc* d, const void* q, const void* k,
                         const void* v, const float* gamma, const float* beta, const float* lambda,
                         const float* h0, const float* g0, float* o, float* h_final, float* g_final,
                         int32_t* steps, float* x_out, const void* workspace, bool lam_full) {
  const mesa_status st = check_desc(d);
  if (st != MESA_OK) return st;
  // a full Lambda is taken by the bf16 kernels at chunk 64, d 64 or 128
  if (lam_full && (d->in_dtype != MESA_BF16 || d->chunk != 64 || (d->dk != 64 && d->dk != 128)))
    return MESA_ERR_UNSUPPORTED;
  const bool any_tokens = d->T > 0;
  if (any_tokens && (!k || !v || !gamma || !beta)) return MESA_ERR_INVALID_ARG;
  if (any_tokens && (phases & kSolve) && (!q || !lambda || !o)) return MESA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, gamma, beta, lambda, h0, g0, o, h_final, g_final, steps, x_out, workspace};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return MESA_ERR_ALIGNMENT;
  return MESA_OK;
}

// the fused preprocessing of a forward call: taps, window, eps, histories
struct FwdPrep {
  const float* wq;
  const float* wk;
  const void* q_hist;
  const void* k_hist;
  int W;
  float inv_eps;
};

mesa_status fwd_impl(int phases, const mesa_fwd_desc* d, const void* q, const void* k,
                     const void* v, const float* gamma, const float* beta, const float* lambda,
                     const float* h0, const float* g0, float* o, float* h_final, float* g_final,
                     int32_t* steps, float* x_out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream, bool lam_full = false, bool warm = false,
                     const FwdPrep* prep = nullptr) {
  const mesa_status st = fwd_validate(phases, d, q, k, v, gamma, beta, lambda, h0, g0, o, h_final, g_final,
                                      steps, x_out, workspace, lam_full);
  if (st != MESA_OK) return st;
  // the warm start is built into the bf16 kernels with a diagonal Lambda
  if (warm && (d->in_dtype != MESA_BF16 || lam_full)) return MESA_ERR_UNSUPPORTED;
  const bool any_tokens = d->T > 0;
  const size_t need = mesa_fwd_workspace_bytes(d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MESA_ERR_WORKSPACE;

  const bool bf16 = d->in_dtype == MESA_BF16;
  const int D = d->dk, C = d->chunk;
  const int BH = d->B * d->H;
  const int NC = (d->T + C - 1) / C;
  const size_t snap = (size_t)BH * NC * mesa::snapshot_bytes(bf16, D);
  void* hb = workspace;
  void* gb = workspace ? static_cast<char*>(workspace) + snap : nullptr;
  int32_t* flags = (workspace && bf16) ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + 2 * snap)
                                       : nullptr;
  // segment states of a split scan follow the snapshots and the flags
  char* segbase = workspace ? static_cast<char*>(workspace) + 2 * snap + (bf16 ? mesa::flag_bytes((size_t)BH * NC) : 0)
                            : nullptr;
  const int NS = mesa::scan_segments(BH, NC, D);
  float* seg_state = (NS > 1 && segbase) ? reinterpret_cast<float*>(segbase) : nullptr;
  float* seg_decay = (NS > 1 && segbase)
                         ? reinterpret_cast<float*>(segbase + (size_t)BH * 2 * (NS - 1) * D * D * 4)
                         : nullptr;

  if ((phases & kScan) && (any_tokens || h_final || g_final)) {
    mesa::ScanParams sp{};
    sp.k = k; sp.v = v; sp.gamma = gamma; sp.beta = beta; sp.h0 = h0; sp.g0 = g0;
    sp.h_final = h_final; sp.g_final = g_final;
    sp.hb = hb; sp.gb = gb;
    sp.BH = BH; sp.T = d->T; sp.NC = NC;
    sp.NS = NS; sp.SEG = mesa::scan_segment_chunks(NC, NS);
    sp.seg_state = seg_state; sp.seg_decay = seg_decay;
    if (prep) {
      sp.prep = 1; sp.W = prep->W; sp.H = d->H; sp.wk = prep->wk; sp.k_hist = prep->k_hist; sp.inv_eps = prep->inv_eps;
    }
    if (mesa::launch_scan(bf16, D, C, sp, stream) != hipSuccess) return MESA_ERR_HIP;
  }
  if ((phases & kSolve) && any_tokens) {
    mesa::CgParams cp{};
    cp.q = q; cp.k = k; cp.v = v; cp.gamma = gamma; cp.beta = beta; cp.lam = lambda;
    cp.hb = hb; cp.gb = gb; cp.o = o; cp.steps = steps; cp.x_out = x_out; cp.unscaled = flags;
    cp.BH = BH; cp.H = d->H; cp.T = d->T; cp.NC = NC; cp.max_steps = d->max_steps;
    cp.tol2 = d->tol > 0.f ? d->tol * d->tol : -1.f;
    cp.lam_full = lam_full ? 1 : 0;
    cp.warm = warm ? 1 : 0;
    if (prep) {
      cp.prep = 1; cp.W = prep->W; cp.wq = prep->wq; cp.wk = prep->wk;
      cp.q_hist = prep->q_hist; cp.k_hist = prep->k_hist; cp.inv_eps = prep->inv_eps;
    }
    if (mesa::launch_cg(bf16, D, C, cp, stream) != hipSuccess) return MESA_ERR_HIP;
  }
  return MESA_OK;
}

}  // namespace

extern "C" {

mesa_status mesa_fwd_chunked(const mesa_fwd_desc* d, const void* q, const void* k, const void* v,
                             const float* gamma, const float* beta, const float* lambda,
                             const float* h0, const float* g0, float* o, float* h_final,
                             float* g_final, int32_t* steps, float* x_out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return fwd_impl(kScan | kSolve, d, q, k, v, gamma, beta, lambda, h0, g0, o, h_final, g_final,
                  steps, x_out, workspace, workspace_bytes, stream);
}

mesa_status mesa_fwd_chunked_warm(const mesa_fwd_desc* d, const void* q, const void* k, const void* v,
                                  const float* gamma, const float* beta, const float* lambda,
                                  const float* h0, const float* g0, float* o, float* h_final,
                                  float* g_final, int32_t* steps, float* x_out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return fwd_impl(kScan | kSolve, d, q, k, v, gamma, beta, lambda, h0, g0, o, h_final, g_final,
                  steps, x_out, workspace, workspace_bytes, stream, false, true);
}

mesa_status mesa_fwd_chunked_prep(const mesa_fwd_desc* d, const void* q_raw, const void* k_raw, const void* v,
                                  const float* w_q, const float* w_k, int32_t window, float eps,
                                  const void* q_hist, const void* k_hist, const float* gamma, const float* beta,
                                  const float* lambda, const float* h0, const float* g0, float* o,
                                  float* h_final, float* g_final, int32_t* steps, float* x_out,
                                  void* q_hist_out, void* k_hist_out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  mesa_status st = fwd_validate(kScan | kSolve, d, q_raw, k_raw, v, gamma, beta, lambda, h0, g0, o, h_final,
                                g_final, steps, x_out, workspace, false);
  if (st != MESA_OK) return st;
  if (window < 1 || !eps_ok(eps) || !w_q || !w_k) return MESA_ERR_INVALID_ARG;
  if (d->in_dtype != MESA_BF16 || d->chunk != 64 || (d->dk != 64 && d->dk != 128) || window > 4)
    return MESA_ERR_UNSUPPORTED;
  const void* ptrs[] = {w_q, w_k, q_hist, k_hist, q_hist_out, k_hist_out};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return MESA_ERR_ALIGNMENT;
  // the next call's histories may not overlap what they are formed from
  const size_t seq_bytes = (size_t)d->B * d->H * d->T * d->dk * 2;
  const size_t hist_bytes = (size_t)d->B * d->H * (window - 1) * d->dk * 2;
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
  };
  const void* ins[] = {q_raw, k_raw, q_hist, k_hist};
  const size_t in_bytes[] = {seq_bytes, seq_bytes, hist_bytes, hist_bytes};
  const void* outs[] = {q_hist_out, k_hist_out};
  for (const void* out : outs)
    for (int b = 0; b < 4; ++b)
      if (overlap(out, hist_bytes, ins[b], in_bytes[b])) return MESA_ERR_INVALID_ARG;
  if (overlap(q_hist_out, hist_bytes, k_hist_out, hist_bytes)) return MESA_ERR_INVALID_ARG;

  const FwdPrep prep{w_q, w_k, q_hist, k_hist, window, 1.0f / eps};
  st = fwd_impl(kScan | kSolve, d, q_raw, k_raw, v, gamma, beta, lambda, h0, g0, o, h_final, g_final, steps,
                x_out, workspace, workspace_bytes, stream, false, false, &prep);
  if (st != MESA_OK || window == 1 || (!q_hist_out && !k_hist_out)) return st;
  mesa::PrepParams pp{};
  pp.x[0] = q_raw; pp.x[1] = k_raw;
  pp.hist_in[0] = q_hist; pp.hist_in[1] = k_hist;
  pp.hist_out[0] = q_hist_out; pp.hist_out[1] = k_hist_out;
  pp.BH = d->B * d->H; pp.H = d->H; pp.T = d->T; pp.W = window; pp.inv_eps = 1.0f / eps;
  return mesa::launch_qk_prep(true, d->dk, pp, stream) == hipSuccess ? MESA_OK : MESA_ERR_HIP;
}

mesa_status mesa_fwd_chunked_ex(const mesa_fwd_desc* d, const void* q, const void* k, const void* v,
                                const float* gamma, const float* beta, const float* lambda,
                                int32_t lambda_full, const float* h0, const float* g0, float* o,
                                float* h_final, float* g_final, int32_t* steps, float* x_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (lambda_full != 0 && lambda_full != 1) return MESA_ERR_INVALID_ARG;
  return fwd_impl(kScan | kSolve, d, q, k, v, gamma, beta, lambda, h0, g0, o, h_final, g_final,
                  steps, x_out, workspace, workspace_bytes, stream, lambda_full != 0);
}

}  // extern "C"

// ---- allocation-free forward ---------------------------------------------------
// Scratch of mesa_fwd_chunked_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends.  In host code `mesa_noalloc_scratch` only
// names the symbol; its device address is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
static __device__ __align__(256) unsigned char mesa_noalloc_scratch[MESA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxNoallocDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxNoallocDevices] = {};

// the scratch address on the current device (looked up on its first use there)
mesa_status noalloc_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MESA_ERR_HIP;
  if (dev < 0 || dev >= kMaxNoallocDevices) return MESA_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MESA_ERR_HIP;
    if (sdev != dev) return MESA_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(mesa_noalloc_scratch)) != hipSuccess || !ptr) return MESA_ERR_HIP;
    g_noalloc_ptr[dev] = ptr;
  }
  *out = g_noalloc_ptr[dev];
  return MESA_OK;
}

}  // namespace

extern "C" {

mesa_status mesa_fwd_chunked_noalloc(const mesa_fwd_desc* d, const void* q, const void* k, const void* v,
                                     const float* gamma, const float* beta, const float* lambda,
                                     const float* h0, const float* g0, float* o, float* h_final,
                                     float* g_final, int32_t* steps, float* x_out, hipStream_t stream) {
  // every host-side check first: no HIP call for a call that cannot run
  const mesa_status st = fwd_validate(kScan | kSolve, d, q, k, v, gamma, beta, lambda, h0, g0, o, h_final,
                                      g_final, steps, x_out, nullptr, false);
  if (st != MESA_OK) return st;
  const size_t need = mesa_fwd_workspace_bytes(d);
  if (need > MESA_NOALLOC_SCRATCH_BYTES) return MESA_ERR_UNSUPPORTED;
  void* scratch = nullptr;
  if (need > 0) {
    const mesa_status sc = noalloc_scratch(stream, &scratch);
    if (sc != MESA_OK) return sc;
  }
  // nothing in the scratch needs clearing: the scan writes every snapshot and
  // segment state before they are read, and the CG kernel writes every chunk's
  // form flag before the strong-decay kernel reads it
  return fwd_impl(kScan | kSolve, d, q, k, v, gamma, beta, lambda, h0, g0, o, h_final, g_final,
                  steps, x_out, scratch, MESA_NOALLOC_SCRATCH_BYTES, stream);
}

mesa_status mesa_fwd_scan(const mesa_fwd_desc* d, const void* k, const void* v, const float* gamma,
                          const float* beta, const float* h0, const float* g0, float* h_final,
                          float* g_final, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return fwd_impl(kScan, d, nullptr, k, v, gamma, beta, nullptr, h0, g0, nullptr, h_final, g_final,
                  nullptr, nullptr, workspace, workspace_bytes, stream);
}

mesa_status mesa_fwd_solve(const mesa_fwd_desc* d, const void* q, const void* k, const void* v,
                           const float* gamma, const float* beta, const float* lambda, float* o,
                           int32_t* steps, float* x_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return fwd_impl(kSolve, d, q, k, v, gamma, beta, lambda, nullptr, nullptr, o, nullptr, nullptr,
                  steps, x_out, workspace, workspace_bytes, stream);
}

namespace {

mesa_status decode_impl(bool symh, bool warm, bool lam_full, int32_t N, int32_t H, int32_t dk, int32_t dv, const void* q,
                        const void* k, const void* v, mesa_dtype in_dtype, const float* gamma,
                        const float* beta, const float* lambda, float* h_state, float* g_state,
                        float* o, int32_t* steps, float* x_out, int32_t max_steps, float tol,
                        hipStream_t stream) {
  if (N < 0 || H < 1 || dk < 1 || dv < 1 || max_steps < 0 || std::isnan(tol)) return MESA_ERR_INVALID_ARG;
  if (in_dtype != MESA_F32 && in_dtype != MESA_BF16) return MESA_ERR_INVALID_ARG;
  if (dk != dv || (dk != 64 && dk != 128)) return MESA_ERR_UNSUPPORTED;
  if ((long long)N * H > (1LL << 31) - 1) return MESA_ERR_UNSUPPORTED;
  if (N == 0) return MESA_OK;
  if (!q || !k || !v || !gamma || !beta || !lambda || !h_state || !g_state || !o || (warm && !x_out))
    return MESA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, gamma, beta, lambda, h_state, g_state, o, steps, x_out};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return MESA_ERR_ALIGNMENT;

  mesa::DecodeParams dp{};
  dp.q = q; dp.k = k; dp.v = v; dp.gamma = gamma; dp.beta = beta; dp.lam = lambda;
  dp.h = h_state; dp.g = g_state; dp.o = o; dp.steps = steps; dp.x_out = x_out;
  dp.x0 = warm ? x_out : nullptr;
  dp.lam_full = lam_full ? 1 : 0;
  dp.P = N * H; dp.H = H; dp.max_steps = max_steps;
  dp.tol2 = tol > 0.f ? tol * tol : -1.f;
  const hipError_t e = mesa::launch_decode(in_dtype == MESA_BF16, dk, symh, warm, dp, stream);
  return e == hipSuccess ? MESA_OK : MESA_ERR_HIP;
}

mesa_status sym_check(int32_t count, int32_t d, const float* a, const float* b) {
  if (count < 0 || d < 1) return MESA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MESA_ERR_UNSUPPORTED;
  if (count == 0) return MESA_OK;
  if (!a || !b) return MESA_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(b)) return MESA_ERR_ALIGNMENT;
  return MESA_OK;
}

}  // namespace

mesa_status mesa_decode_step(int32_t N, int32_t H, int32_t dk, int32_t dv, const void* q,
                             const void* k, const void* v, mesa_dtype in_dtype, const float* gamma,
                             const float* beta, const float* lambda, float* h_state,
                             float* g_state, float* o, int32_t* steps, float* x_out,
                             int32_t max_steps, float tol, hipStream_t stream) {
  return decode_impl(false, false, false, N, H, dk, dv, q, k, v, in_dtype, gamma, beta, lambda, h_state, g_state, o,
                     steps, x_out, max_steps, tol, stream);
}

mesa_status mesa_decode_step_symh(int32_t N, int32_t H, int32_t dk, int32_t dv, const void* q,
                                  const void* k, const void* v, mesa_dtype in_dtype, const float* gamma,
                                  const float* beta, const float* lambda, float* h_sym,
                                  float* g_state, float* o, int32_t* steps, float* x_out,
                                  int32_t max_steps, float tol, hipStream_t stream) {
  return decode_impl(true, false, false, N, H, dk, dv, q, k, v, in_dtype, gamma, beta, lambda, h_sym, g_state, o,
                     steps, x_out, max_steps, tol, stream);
}

mesa_status mesa_decode_step_warm(int32_t N, int32_t H, int32_t dk, int32_t dv, const void* q,
                                  const void* k, const void* v, mesa_dtype in_dtype, const float* gamma,
                                  const float* beta, const float* lambda, float* h_state, int32_t h_packed,
                                  float* g_state, float* x_state, float* o, int32_t* steps,
                                  int32_t max_steps, float tol, hipStream_t stream) {
  if (h_packed != 0 && h_packed != 1) return MESA_ERR_INVALID_ARG;
  return decode_impl(h_packed == 1, true, false, N, H, dk, dv, q, k, v, in_dtype, gamma, beta, lambda, h_state,
                     g_state, o, steps, x_state, max_steps, tol, stream);
}

mesa_status mesa_decode_step_ex(int32_t N, int32_t H, int32_t dk, int32_t dv, const void* q, const void* k,
                                const void* v, mesa_dtype in_dtype, const float* gamma, const float* beta,
                                const float* lambda, int32_t lambda_full, float* h_state, int32_t h_packed,
                                float* g_state, float* x_state, float* o, int32_t* steps, float* x_out,
                                int32_t max_steps, float tol, hipStream_t stream) {
  if (h_packed != 0 && h_packed != 1) return MESA_ERR_INVALID_ARG;
  if (lambda_full != 0 && lambda_full != 1) return MESA_ERR_INVALID_ARG;
  if (x_state && x_out) return MESA_ERR_INVALID_ARG;  // a warm step returns its solution in x_state
  return decode_impl(h_packed == 1, x_state != nullptr, lambda_full == 1, N, H, dk, dv, q, k, v, in_dtype, gamma,
                     beta, lambda, h_state, g_state, o, steps, x_state ? x_state : x_out, max_steps, tol, stream);
}

}  // extern "C"

namespace {

mesa_status check_bwd(const mesa_fwd_desc* d) {
  const mesa_status st = check_desc(d);
  if (st != MESA_OK) return st;
  if (d->in_dtype != MESA_BF16 || (d->dk != 64 && d->dk != 128) || d->chunk != 64) return MESA_ERR_UNSUPPORTED;
  return MESA_OK;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

struct BwdLayout {
  size_t fwd, rhs, nu, yn, snap, lam, seg, segdec, lamf, total;
  int NS, SEG;
};

BwdLayout bwd_layout(const mesa_fwd_desc* d) {
  BwdLayout L{};
  const size_t BH = (size_t)d->B * d->H, T = (size_t)d->T, D = (size_t)d->dk;
  const size_t NC = (T + d->chunk - 1) / d->chunk;
  size_t off = align256(mesa_fwd_workspace_bytes(d));
  L.fwd = 0;
  L.rhs = off; off = align256(off + BH * T * D * 2);
  L.nu = off; off = align256(off + BH * T * 4);
  L.yn = off; off = align256(off + BH * T * D * 4);
  L.snap = off; off = align256(off + 2 * BH * NC * D * D * 2);
  L.NS = mesa::bwd_scan_segments((long long)BH, (int)NC, (int)D);
  L.SEG = NC > 0 ? (int)((NC + L.NS - 1) / L.NS) : 0;
  L.lam = off; off = align256(off + BH * L.NS * D * 4);
  L.seg = off; off = align256(off + BH * 2 * (L.NS - 1) * D * D * 4);
  L.segdec = off; off = align256(off + BH * (L.NS - 1) * 4);
  L.lamf = off; off = align256(off + (size_t)d->H * mesa::kLamSplits * D * D * 4);  // full-Lambda partial sums
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t mesa_bwd_workspace_bytes(const mesa_fwd_desc* d) {
  if (check_bwd(d) != MESA_OK) return 0;
  return bwd_layout(d).total;
}

}  // extern "C"

namespace {

mesa_status bwd_impl(const mesa_fwd_desc* d, const void* q, const void* k, const void* v,
                     const float* gamma, const float* beta, const float* lambda, bool lam_full,
                     const float* h0, const float* g0, const float* x, const float* d_o,
                     const float* d_hfinal, const float* d_gfinal,
                     float* dq, float* dk, float* dv, float* dgamma, float* dbeta,
                     float* dlambda, float* dh0, float* dg0, int32_t* adj_steps,
                     int32_t states_in_workspace, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  const mesa_status st = check_bwd(d);
  if (st != MESA_OK) return st;
  if (states_in_workspace != 0 && states_in_workspace != 1) return MESA_ERR_INVALID_ARG;
  const bool any = d->T > 0;
  if (!lambda || !dlambda) return MESA_ERR_INVALID_ARG;
  if (any && (!q || !k || !v || !gamma || !beta || !x || !d_o || !dq || !dk || !dv || !dgamma || !dbeta))
    return MESA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, gamma, beta, lambda, h0, g0, x, d_o, d_hfinal, d_gfinal,
                        dq, dk, dv, dgamma, dbeta, dlambda, dh0, dg0, adj_steps, workspace};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return MESA_ERR_ALIGNMENT;
  const BwdLayout L = bwd_layout(d);
  if (!workspace || workspace_bytes < L.total) return MESA_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  const int D = d->dk, C = d->chunk, BH = d->B * d->H;
  const int NC = (d->T + C - 1) / C;
  // 1. the forward's boundary states, into the forward part of the workspace
  //    (unless the forward call left them there)
  if (any && !states_in_workspace) {
    const mesa_status s1 = fwd_impl(kScan, d, nullptr, k, v, gamma, beta, nullptr, h0, g0, nullptr, nullptr,
                                    nullptr, nullptr, nullptr, ws, mesa_fwd_workspace_bytes(d), stream);
    if (s1 != MESA_OK) return s1;
  }
  const size_t snap = (size_t)BH * NC * mesa::snapshot_bytes(true, D);
  mesa::BwdParams bp{};
  bp.k = k; bp.v = v; bp.gamma = gamma; bp.beta = beta;
  bp.hb = ws; bp.gb = ws + snap;
  bp.x = x; bp.d_o = d_o; bp.d_hfinal = d_hfinal; bp.d_gfinal = d_gfinal;
  bp.rhs = ws + L.rhs;
  bp.nu = reinterpret_cast<float*>(ws + L.nu);
  bp.yn = reinterpret_cast<float*>(ws + L.yn);
  const size_t sn = (size_t)BH * NC * D * D;
  bp.snap_r = reinterpret_cast<uint16_t*>(ws + L.snap);
  bp.snap_s = bp.snap_r + sn;
  bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.dbeta = dbeta; bp.dgamma = dgamma;
  bp.lam_part = reinterpret_cast<float*>(ws + L.lam);
  bp.dlam = dlambda; bp.dh0 = dh0; bp.dg0 = dg0;
  bp.seg_state = reinterpret_cast<float*>(ws + L.seg);
  bp.seg_decay = reinterpret_cast<float*>(ws + L.segdec);
  bp.BH = BH; bp.H = d->H; bp.T = d->T; bp.NC = NC; bp.NS = L.NS; bp.SEG = L.SEG;
  bp.lam_full = lam_full ? 1 : 0;
  bp.lam_full_part = reinterpret_cast<float*>(ws + L.lamf);
  if (any) {
    // 2. right-hand sides of the adjoint systems
    if (mesa::launch_bwd(0, D, bp, stream) != hipSuccess) return MESA_ERR_HIP;
    // 3. adjoint solves by the forward CG (solutions only)
    mesa::CgParams cp{};
    cp.q = bp.rhs; cp.k = k; cp.v = v; cp.gamma = gamma; cp.beta = beta; cp.lam = lambda;
    cp.hb = bp.hb; cp.gb = bp.gb; cp.o = nullptr; cp.steps = adj_steps;
    cp.x_out = reinterpret_cast<float*>(ws + L.yn);
    cp.unscaled = reinterpret_cast<int32_t*>(ws + 2 * snap);
    cp.BH = BH; cp.H = d->H; cp.T = d->T; cp.NC = NC; cp.max_steps = d->max_steps;
    cp.tol2 = d->tol > 0.f ? d->tol * d->tol : -1.f;
    cp.lam_full = lam_full ? 1 : 0;
    if (mesa::launch_cg(true, D, C, cp, stream) != hipSuccess) return MESA_ERR_HIP;
  }
  // 4. adjoint scan (also the initial-state gradients); 5. per-token gradients and dlambda
  if ((any || dh0 || dg0) && mesa::launch_bwd(1, D, bp, stream) != hipSuccess) return MESA_ERR_HIP;
  if (mesa::launch_bwd(2, D, bp, stream) != hipSuccess) return MESA_ERR_HIP;
  return MESA_OK;
}

}  // namespace

extern "C" {

mesa_status mesa_bwd_chunked(const mesa_fwd_desc* d, const void* q, const void* k, const void* v,
                             const float* gamma, const float* beta, const float* lambda,
                             const float* h0, const float* g0, const float* x, const float* d_o,
                             const float* d_hfinal, const float* d_gfinal,
                             float* dq, float* dk, float* dv, float* dgamma, float* dbeta,
                             float* dlambda, float* dh0, float* dg0, int32_t* adj_steps,
                             int32_t states_in_workspace, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  return bwd_impl(d, q, k, v, gamma, beta, lambda, false, h0, g0, x, d_o, d_hfinal, d_gfinal, dq, dk, dv,
                  dgamma, dbeta, dlambda, dh0, dg0, adj_steps, states_in_workspace, workspace,
                  workspace_bytes, stream);
}

mesa_status mesa_bwd_chunked_ex(const mesa_fwd_desc* d, const void* q, const void* k, const void* v,
                                const float* gamma, const float* beta, const float* lambda,
                                int32_t lambda_full, const float* h0, const float* g0, const float* x,
                                const float* d_o, const float* d_hfinal, const float* d_gfinal,
                                float* dq, float* dk, float* dv, float* dgamma, float* dbeta,
                                float* dlambda, float* dh0, float* dg0, int32_t* adj_steps,
                                int32_t states_in_workspace, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (lambda_full != 0 && lambda_full != 1) return MESA_ERR_INVALID_ARG;
  return bwd_impl(d, q, k, v, gamma, beta, lambda, lambda_full == 1, h0, g0, x, d_o, d_hfinal, d_gfinal, dq,
                  dk, dv, dgamma, dbeta, dlambda, dh0, dg0, adj_steps, states_in_workspace, workspace,
                  workspace_bytes, stream);
}

mesa_status mesa_qk_preprocess(int32_t B, int32_t H, int32_t T, int32_t d, int32_t window,
                               mesa_dtype dtype, const void* q_raw, const void* k_raw,
                               const float* w_q, const float* w_k, const void* q_hist,
                               const void* k_hist, float eps, void* q_out, void* k_out,
                               void* q_hist_out, void* k_hist_out, hipStream_t stream) {
  if (B < 0 || H < 1 || T < 0 || window < 1 || !eps_ok(eps)) return MESA_ERR_INVALID_ARG;
  if (dtype != MESA_F32 && dtype != MESA_BF16) return MESA_ERR_INVALID_ARG;
  if ((d != 16 && d != 64 && d != 128) || window > 4) return MESA_ERR_UNSUPPORTED;
  if ((long long)B * H > 65535) return MESA_ERR_UNSUPPORTED;
  if (B == 0) return MESA_OK;
  const size_t esz = dtype == MESA_BF16 ? 2 : 4;
  const size_t seq_bytes = (size_t)B * H * T * d * esz;
  const size_t hist_bytes = (size_t)B * H * (window - 1) * d * esz;
  if ((T > 0 && (!q_raw || !k_raw || !q_out || !k_out)) || !w_q || !w_k) return MESA_ERR_INVALID_ARG;
  const void* ptrs[] = {q_raw, k_raw, w_q, w_k, q_hist, k_hist, q_out, k_out, q_hist_out, k_hist_out};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return MESA_ERR_ALIGNMENT;
  // outputs may not overlap the inputs they are computed from
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
  };
  const void* ins[] = {q_raw, k_raw, q_hist, k_hist};
  const size_t in_bytes[] = {seq_bytes, seq_bytes, hist_bytes, hist_bytes};
  const void* outs[] = {q_out, k_out, q_hist_out, k_hist_out};
  const size_t out_bytes[] = {seq_bytes, seq_bytes, hist_bytes, hist_bytes};
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 4; ++b)
      if (overlap(outs[a], out_bytes[a], ins[b], in_bytes[b])) return MESA_ERR_INVALID_ARG;

  mesa::PrepParams pp{};
  pp.x[0] = q_raw; pp.x[1] = k_raw; pp.w[0] = w_q; pp.w[1] = w_k;
  pp.hist_in[0] = q_hist; pp.hist_in[1] = k_hist;
  pp.out[0] = q_out; pp.out[1] = k_out;
  pp.hist_out[0] = q_hist_out; pp.hist_out[1] = k_hist_out;
  pp.BH = B * H; pp.H = H; pp.T = T; pp.W = window; pp.inv_eps = 1.0f / eps;
  return mesa::launch_qk_prep(dtype == MESA_BF16, d, pp, stream) == hipSuccess ? MESA_OK : MESA_ERR_HIP;
}

size_t mesa_sym_state_floats(int32_t d) {
  if (d != 64 && d != 128) return 0;
  return mesa::sym_state_floats(d);
}

mesa_status mesa_sym_pack(int32_t count, int32_t d, const float* full, float* packed, hipStream_t stream) {
  const mesa_status st = sym_check(count, d, full, packed);
  if (st != MESA_OK || count == 0) return st;
  return mesa::launch_sym_pack(d, count, full, packed, stream) == hipSuccess ? MESA_OK : MESA_ERR_HIP;
}

mesa_status mesa_sym_unpack(int32_t count, int32_t d, const float* packed, float* full, hipStream_t stream) {
  const mesa_status st = sym_check(count, d, packed, full);
  if (st != MESA_OK || count == 0) return st;
  return mesa::launch_sym_unpack(d, count, packed, full, stream) == hipSuccess ? MESA_OK : MESA_ERR_HIP;
}

}  // extern "C"
