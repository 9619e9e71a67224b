// Host side of the libmoc C ABI: argument validation, workspace sizing and carving, launches.
// Every check runs before anything is enqueued; no C++ exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "moc.h"
#include "moc_params.h"


namespace moc_host {
hipError_t launch_pool(const moc_layout* lay, const void* K, float* kbar, hipStream_t st);
hipError_t launch_route(const moc_layout* lay, const moc::RouteParams& p, const void* Q,
                        const float* kbar, int32_t* sel, int32_t* nsel, void* ws, hipStream_t st);
size_t route_workspace(const moc_layout* lay);
size_t route_noalloc_limit();
void* route_noalloc_scratch(hipError_t* err);
size_t outer_workspace(const moc_layout* lay);
hipError_t launch_route_outer(const moc_layout* lay, const int32_t* seg_chunk, int nseg, int M,
                              int causal, const void* Q, const void* K, int32_t* seg_sel,
                              int32_t* seg_nsel, uint32_t* cmask, void* ws, hipStream_t st);
hipError_t launch_varlen(const moc_layout* lay, const moc::VarlenParams& p, const int32_t* sel,
                         const int32_t* nsel, int32_t* counts, int32_t* totals,
                         int32_t* tile_base, const moc_varlen* out, int64_t* pair_count,
                         hipStream_t st);
hipError_t launch_attn_fwd(const moc_layout* lay, const moc_varlen* vl, const void* Q,
                           const void* K, const void* V, float scale, void* O, float* lse,
                           float* pO, float* plse, void* vt_ws, hipStream_t st);
size_t attn_fwd_vt_bytes(const moc_layout* lay);
hipError_t launch_attn_fwd_mx(const moc_layout* lay, const moc_varlen* vl, const uint8_t* Qc,
                              const uint8_t* Qs, const uint8_t* Kc, const uint8_t* Ks,
                              const void* V, float scale, void* O, float* lse, float* pO,
                              float* plse, void* vt_ws, hipStream_t st);
hipError_t launch_mx_quantize(const moc_layout* lay, const void* X, uint8_t* codes,
                              uint8_t* scales, hipStream_t st);
size_t mx_quantize_v_bytes(const moc_layout* lay);
hipError_t launch_mx_quantize_v(const moc_layout* lay, const void* V, uint8_t* out,
                                hipStream_t st);
hipError_t launch_attn_fwd_mxv(const moc_layout* lay, const moc_varlen* vl, const uint8_t* Qc,
                               const uint8_t* Qs, const uint8_t* Kc, const uint8_t* Ks,
                               const uint8_t* Vq, float scale, void* O, float* lse, float* pO,
                               float* plse, hipStream_t st);
hipError_t launch_attn_bwd(const moc_layout* lay, const moc_varlen* vl, const void* Q,
                           const void* K, const void* V, const void* O, const float* lse,
                           const void* dO, float scale, void* dQ, void* dK, void* dV,
                           void* ws, size_t ws_bytes, hipStream_t st);
size_t attn_bwd_workspace(const moc_layout* lay, int64_t routed_rows);
hipError_t launch_varlen_guard(const moc_layout* lay, const moc_varlen* vl, hipStream_t st);
int attn_tile_rows();
int attn_bwd_key_rows();
int attn_bwd_text_split(int L);
hipError_t launch_layout_check(const moc_layout* lay, hipStream_t st);
uint32_t layout_check_host(const int32_t* off, const int32_t* shot, int C, int L, int tb, int te);
}  // namespace moc_host

namespace {

constexpr int kInvTile = 256;    // queries per inversion tile
constexpr size_t kAlign = 256;

thread_local std::string g_last_error;

moc_status fail(moc_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = std::string(moc_status_string(s)) + ": " + buf;
  return s;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

moc_status check_layout(const moc_layout* lay) {
  if (!lay) return fail(MOC_EINVAL, "layout is NULL");
  if (lay->dtype != MOC_F32 && lay->dtype != MOC_BF16)
    return fail(MOC_EDTYPE, "dtype %d is neither MOC_F32 nor MOC_BF16", lay->dtype);
  if (lay->B < 1 || lay->H < 1 || lay->L < 1)
    return fail(MOC_ESHAPE, "B, H, L must be >= 1 (got %d, %d, %d)", lay->B, lay->H, lay->L);
  if (lay->d != 64 && lay->d != 128) return fail(MOC_ESHAPE, "d must be 64 or 128 (got %d)", lay->d);
  if (lay->C < 1 || lay->C > MOC_MAX_C || lay->C > lay->L)
    return fail(MOC_ESHAPE, "C must be in [1, min(L, %d)] (got %d)", MOC_MAX_C, lay->C);
  if (!lay->chunk_offsets || !lay->chunk_shot) return fail(MOC_EINVAL, "layout arrays are NULL");
  if (lay->text_begin < 0 || lay->text_end < lay->text_begin || lay->text_end > lay->L)
    return fail(MOC_EINVAL, "text range [%d, %d) outside [0, %d]", lay->text_begin, lay->text_end,
                lay->L);
  const int64_t elems = static_cast<int64_t>(lay->B) * lay->H * lay->L * lay->d;
  if (elems >= (int64_t(1) << 40)) return fail(MOC_ESHAPE, "tensor too large");
  return MOC_OK;
}

int k_eff_of(const moc_route_cfg* cfg, int C) { return cfg->top_k < C ? cfg->top_k : C; }

moc_status check_cfg(const moc_layout* lay, const moc_route_cfg* cfg) {
  if (!cfg) return fail(MOC_EINVAL, "route cfg is NULL");
  if (cfg->top_k < 0) return fail(MOC_EINVAL, "top_k must be >= 0 (got %d)", cfg->top_k);
  if (cfg->causal != 0 && cfg->causal != 1) return fail(MOC_EINVAL, "causal must be 0 or 1");
  if (k_eff_of(cfg, lay->C) > MOC_MAX_TOPK)
    return fail(MOC_ESHAPE, "min(top_k, C) = %d exceeds %d", k_eff_of(cfg, lay->C), MOC_MAX_TOPK);
  if (!(cfg->p_max >= 0.f && cfg->p_max <= 1.f))
    return fail(MOC_EINVAL, "p_max must be in [0, 1]");
  if (!(cfg->lambda >= 0.f) || !std::isfinite(cfg->lambda))
    return fail(MOC_EINVAL, "lambda must be finite and >= 0");
  if (cfg->max_drop_in < 0 || cfg->max_drop_in > MOC_MAX_DROP_IN)
    return fail(MOC_ESHAPE, "max_drop_in must be in [0, %d]", MOC_MAX_DROP_IN);
  const int S = moc_sel_width(cfg, lay->C);
  const int64_t rows = static_cast<int64_t>(lay->B) * lay->H * lay->L * (S > 0 ? S : 1);
  if (rows >= (int64_t(1) << 31)) return fail(MOC_ESHAPE, "B*H*L*S must be < 2^31");
  return MOC_OK;
}

struct VarlenSizes {
  size_t counts, totals, tile_base, bucket_off, bucket_q, slot, rtiles, n_rtiles, atiles, n_atiles,
      ktiles, n_ktiles, status;
  int max_rtiles, max_atiles, max_ktiles, n_text_split, nqt;
  size_t total() const {
    return counts + totals + tile_base + bucket_off + bucket_q + slot + rtiles + n_rtiles + atiles +
           n_atiles + ktiles + n_ktiles + status;
  }
};

VarlenSizes varlen_sizes(const moc_layout* lay, int S) {
  VarlenSizes z;
  const int64_t BH = static_cast<int64_t>(lay->B) * lay->H;
  const int64_t NB = BH * lay->C;
  const int64_t sel = BH * lay->L * S;
  z.nqt = (lay->L + kInvTile - 1) / kInvTile;
  z.max_rtiles = static_cast<int>((sel + moc_host::attn_tile_rows() - 1) / moc_host::attn_tile_rows() + NB);
  z.max_atiles = (lay->L + moc_host::attn_tile_rows() - 1) / moc_host::attn_tile_rows() + lay->C + 1;
  z.counts = align_up(sizeof(int32_t) * NB * z.nqt);
  z.totals = align_up(sizeof(int32_t) * NB);
  z.tile_base = align_up(sizeof(int32_t) * NB);
  z.bucket_off = align_up(sizeof(int32_t) * (NB + 1));
  z.bucket_q = align_up(sizeof(int32_t) * (sel > 0 ? sel : 1));
  z.slot = align_up(sizeof(int32_t) * (sel > 0 ? sel : 1));
  z.rtiles = align_up(sizeof(int32_t) * 2 * z.max_rtiles);
  z.n_rtiles = kAlign;
  z.atiles = align_up(sizeof(int32_t) * 6 * z.max_atiles);
  z.n_atiles = kAlign;
  const int KR = moc_host::attn_bwd_key_rows();
  const int text = lay->text_end - lay->text_begin;
  z.n_text_split = moc_host::attn_bwd_text_split(lay->L);
  z.max_ktiles = (lay->L + KR - 1) / KR + lay->C + (text + KR - 1) / KR * z.n_text_split;
  z.ktiles = align_up(sizeof(int32_t) * 6 * z.max_ktiles);
  z.n_ktiles = kAlign;
  z.status = kAlign;
  return z;
}

// routed (query, chunk) rows of the static bound: every query of every (b, h) routed S times
int64_t routed_max_of(const moc_layout* lay, int S) {
  return static_cast<int64_t>(lay->B) * lay->H * lay->L * S;
}

// FWD workspace: partial output rows and their LSE for `rows` routed rows, then V^T
size_t fwd_bytes(const moc_layout* lay, int64_t rows) {
  const int64_t r = rows > 0 ? rows : 1;
  return align_up(sizeof(float) * r * lay->d) + align_up(sizeof(float) * r) +
         align_up(moc_host::attn_fwd_vt_bytes(lay));
}

moc_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOC_OK;
  return fail(MOC_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// With moc_layout.check set, every entry point first enqueues the layout check kernel; the
// call's kernels then skip their work if the word is non-zero.
moc_status run_layout_check(const moc_layout* lay, void* stream) {
  if (!lay->check) return MOC_OK;
  return hip_status(moc_host::launch_layout_check(lay, static_cast<hipStream_t>(stream)),
                    "layout check launch");
}

}  // namespace

extern "C" {

const char* moc_status_string(moc_status s) {
  switch (s) {
    case MOC_OK: return "MOC_OK";
    case MOC_EINVAL: return "MOC_EINVAL";
    case MOC_ESHAPE: return "MOC_ESHAPE";
    case MOC_EDTYPE: return "MOC_EDTYPE";
    case MOC_EWORKSPACE: return "MOC_EWORKSPACE";
    case MOC_EUNSUPPORTED: return "MOC_EUNSUPPORTED";
    case MOC_EHIP: return "MOC_EHIP";
    case MOC_EINTERNAL: return "MOC_EINTERNAL";
    case MOC_ELAYOUT: return "MOC_ELAYOUT";
  }
  return "MOC_UNKNOWN";
}

const char* moc_last_error(void) { return g_last_error.c_str(); }

int32_t moc_sel_width(const moc_route_cfg* cfg, int32_t C) {
  if (!cfg || C < 1) return 0;
  const int k = cfg->top_k < 0 ? 0 : (cfg->top_k < C ? cfg->top_k : C);
  return k + (cfg->lambda > 0.f ? cfg->max_drop_in : 0);
}

moc_status moc_poisson_thresholds(float lambda, int32_t max_drop_in, uint64_t* thr) {
  if (!thr) return fail(MOC_EINVAL, "thr is NULL");
  if (max_drop_in < 0 || max_drop_in > MOC_MAX_DROP_IN)
    return fail(MOC_ESHAPE, "max_drop_in must be in [0, %d]", MOC_MAX_DROP_IN);
  if (!(lambda >= 0.f) || !std::isfinite(lambda)) return fail(MOC_EINVAL, "bad lambda");
  // CDF of Poisson(lambda) accumulated term by term in binary64, in the order written.
  const double lam = static_cast<double>(lambda);
  double term = std::exp(-lam);
  double cdf = term;
  for (int i = 0; i < max_drop_in; ++i) {
    if (i > 0) {
      term = term * lam / static_cast<double>(i);
      cdf = cdf + term;
    }
    double v = std::floor(cdf * 4294967296.0);
    uint64_t u = static_cast<uint64_t>(v);
    thr[i] = u > (uint64_t(1) << 32) ? (uint64_t(1) << 32) : u;
  }
  return MOC_OK;
}

size_t moc_workspace_bytes(const moc_layout* lay, const moc_route_cfg* cfg, int32_t op) {
  if (check_layout(lay) != MOC_OK) return 0;
  if (check_cfg(lay, cfg) != MOC_OK) return 0;
  const int S = moc_sel_width(cfg, lay->C);
  switch (op) {
    case MOC_OP_ROUTE: return moc_host::route_workspace(lay);
    case MOC_OP_VARLEN: return varlen_sizes(lay, S).total();
    case MOC_OP_FWD: return fwd_bytes(lay, routed_max_of(lay, S));
    case MOC_OP_BWD: return moc_host::attn_bwd_workspace(lay, routed_max_of(lay, S));
    case MOC_OP_OUTER: return moc_host::outer_workspace(lay);
    default: fail(MOC_EINVAL, "unknown op %d", op); return 0;
  }
}

moc_status moc_pool_keys(const moc_layout* lay, const void* K, float* kbar, void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    if (!K || !kbar) return fail(MOC_EINVAL, "K or kbar is NULL");
    if (static_cast<const void*>(kbar) == K) return fail(MOC_EINVAL, "kbar aliases K");
    if ((s = run_layout_check(lay, stream)) != MOC_OK) return s;
    return hip_status(moc_host::launch_pool(lay, K, kbar, static_cast<hipStream_t>(stream)),
                      "pool launch");
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_pool_keys");
  }
}

namespace {
moc_status route_impl(const moc_layout* lay, const moc_route_cfg* cfg, const void* Q,
                      const float* kbar, const uint32_t* cmask, int32_t* sel, int32_t* nsel,
                      void* ws, size_t ws_bytes, void* stream) {
  moc_status s = check_layout(lay);
  if (s != MOC_OK) return s;
  s = check_cfg(lay, cfg);
  if (s != MOC_OK) return s;
  const int S = moc_sel_width(cfg, lay->C);
  if (!Q || !kbar || !nsel || (S > 0 && !sel)) return fail(MOC_EINVAL, "NULL tensor argument");
  if (static_cast<void*>(sel) == static_cast<void*>(nsel) && S > 0)
    return fail(MOC_EINVAL, "sel aliases nsel");
  const size_t need = moc_host::route_workspace(lay);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOC_EWORKSPACE, "ROUTE workspace needs %zu bytes (got %zu)", need,
                ws ? ws_bytes : size_t(0));
  moc::RouteParams p;
  std::memset(&p, 0, sizeof(p));
  p.B = lay->B; p.H = lay->H; p.L = lay->L; p.C = lay->C; p.S = S;
  p.k_eff = k_eff_of(cfg, lay->C);
  p.causal = cfg->causal;
  p.drop_off = cfg->p_max > 0.f ? 1 : 0;
  p.drop_in = cfg->lambda > 0.f ? 1 : 0;
  p.m_cap = p.drop_in ? cfg->max_drop_in : 0;
  p.p_max = cfg->p_max;
  p.seed = cfg->seed;
  p.cmask = cmask;
  p.cmask_w = (lay->C + 31) / 32;
  p.chk = lay->check;
  if (p.drop_in) {
    s = moc_poisson_thresholds(cfg->lambda, cfg->max_drop_in, p.thr);
    if (s != MOC_OK) return s;
  }
  if ((s = run_layout_check(lay, stream)) != MOC_OK) return s;
  return hip_status(moc_host::launch_route(lay, p, Q, kbar, sel, nsel, ws,
                                           static_cast<hipStream_t>(stream)),
                    "route launch");
}
}  // namespace

moc_status moc_route(const moc_layout* lay, const moc_route_cfg* cfg, const void* Q,
                     const float* kbar, int32_t* sel, int32_t* nsel, void* ws, size_t ws_bytes,
                     void* stream) {
  try {
    return route_impl(lay, cfg, Q, kbar, nullptr, sel, nsel, ws, ws_bytes, stream);
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_route");
  }
}

moc_status moc_route_noalloc(const moc_layout* lay, const moc_route_cfg* cfg, const void* Q,
                             const float* kbar, int32_t* sel, int32_t* nsel, void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    const size_t need = moc_host::route_workspace(lay);
    if (need > moc_host::route_noalloc_limit())
      return fail(MOC_ESHAPE,
                  "moc_route_noalloc: B*H*C*d*6 = %zu bytes of scratch exceed its %zu-byte "
                  "static buffer (use moc_route with a workspace)",
                  need, moc_host::route_noalloc_limit());
    void* ws = nullptr;
    if (need > 0) {
      hipError_t e = hipSuccess;
      ws = moc_host::route_noalloc_scratch(&e);
      if (!ws) return hip_status(e == hipSuccess ? hipErrorUnknown : e, "scratch lookup");
    }
    return route_impl(lay, cfg, Q, kbar, nullptr, sel, nsel, ws, need, stream);
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_route_noalloc");
  }
}

moc_status moc_route_masked(const moc_layout* lay, const moc_route_cfg* cfg, const void* Q,
                            const float* kbar, const uint32_t* cand_mask, int32_t* sel,
                            int32_t* nsel, void* ws, size_t ws_bytes, void* stream) {
  try {
    if (!cand_mask) return fail(MOC_EINVAL, "cand_mask is NULL");
    return route_impl(lay, cfg, Q, kbar, cand_mask, sel, nsel, ws, ws_bytes, stream);
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_route_masked");
  }
}

moc_status moc_route_outer(const moc_layout* lay, const int32_t* seg_chunk, int32_t nseg,
                           int32_t M, int32_t causal, const void* Q, const void* K,
                           int32_t* seg_sel, int32_t* seg_nsel, uint32_t* cand_mask, void* ws,
                           size_t ws_bytes, void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    if (nseg < 1 || nseg > MOC_MAX_SEG || nseg > lay->C)
      return fail(MOC_ESHAPE, "nseg must be in [1, min(C, %d)] (got %d)", MOC_MAX_SEG, nseg);
    if (M < 0) return fail(MOC_EINVAL, "M must be >= 0 (got %d)", M);
    const int Ms = M < nseg ? M : nseg;
    if (Ms > MOC_MAX_TOPM)
      return fail(MOC_ESHAPE, "min(M, nseg) = %d exceeds %d", Ms, MOC_MAX_TOPM);
    if (causal != 0 && causal != 1) return fail(MOC_EINVAL, "causal must be 0 or 1");
    if (!seg_chunk || !Q || !K || !seg_nsel || !cand_mask || (Ms > 0 && !seg_sel))
      return fail(MOC_EINVAL, "NULL argument");
    const size_t need = moc_host::outer_workspace(lay);
    if (!ws || ws_bytes < need)
      return fail(MOC_EWORKSPACE, "OUTER workspace needs %zu bytes (got %zu)", need,
                  ws ? ws_bytes : size_t(0));
    if ((s = run_layout_check(lay, stream)) != MOC_OK) return s;
    return hip_status(moc_host::launch_route_outer(lay, seg_chunk, nseg, M, causal, Q, K,
                                                   seg_sel, seg_nsel, cand_mask, ws,
                                                   static_cast<hipStream_t>(stream)),
                      "outer route launch");
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_route_outer");
  }
}

moc_status moc_build_varlen(const moc_layout* lay, const moc_route_cfg* cfg, const int32_t* sel,
                            const int32_t* nsel, moc_varlen* out, int64_t* pair_count, void* ws,
                            size_t ws_bytes, void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    s = check_cfg(lay, cfg);
    if (s != MOC_OK) return s;
    const int S = moc_sel_width(cfg, lay->C);
    if (!nsel || !out || !pair_count || (S > 0 && !sel))
      return fail(MOC_EINVAL, "NULL argument");
    const VarlenSizes z = varlen_sizes(lay, S);
    if (!ws || ws_bytes < z.total())
      return fail(MOC_EWORKSPACE, "VARLEN workspace needs %zu bytes (got %zu)", z.total(),
                  ws ? ws_bytes : size_t(0));
    char* w = static_cast<char*>(ws);
    int32_t* counts = reinterpret_cast<int32_t*>(w); w += z.counts;
    int32_t* totals = reinterpret_cast<int32_t*>(w); w += z.totals;
    int32_t* tile_base = reinterpret_cast<int32_t*>(w); w += z.tile_base;
    out->bucket_off = reinterpret_cast<int32_t*>(w); w += z.bucket_off;
    out->bucket_q = reinterpret_cast<int32_t*>(w); w += z.bucket_q;
    out->slot = reinterpret_cast<int32_t*>(w); w += z.slot;
    out->rtiles = reinterpret_cast<int32_t*>(w); w += z.rtiles;
    out->n_rtiles = reinterpret_cast<int32_t*>(w); w += z.n_rtiles;
    out->atiles = reinterpret_cast<int32_t*>(w); w += z.atiles;
    out->n_atiles = reinterpret_cast<int32_t*>(w); w += z.n_atiles;
    out->ktiles = reinterpret_cast<int32_t*>(w); w += z.ktiles;
    out->n_ktiles = reinterpret_cast<int32_t*>(w); w += z.n_ktiles;
    out->status = reinterpret_cast<uint32_t*>(w); w += z.status;
    out->routed_max = routed_max_of(lay, S);
    out->routed_cap = out->routed_max;
    out->max_ktiles = z.max_ktiles;
    out->n_text_split = z.n_text_split;
    out->scratch = counts;
    out->S = S;
    out->tile_rows = moc_host::attn_tile_rows();
    out->max_rtiles = z.max_rtiles;
    out->max_atiles = z.max_atiles;
    moc::VarlenParams p;
    p.B = lay->B; p.H = lay->H; p.L = lay->L; p.C = lay->C; p.S = S; p.nqt = z.nqt;
    p.tile_rows = moc_host::attn_tile_rows(); p.max_rtiles = z.max_rtiles; p.max_atiles = z.max_atiles;
    p.text_begin = lay->text_begin; p.text_end = lay->text_end;
    p.key_rows = moc_host::attn_bwd_key_rows(); p.max_ktiles = z.max_ktiles;
    p.n_text_split = z.n_text_split;
    p.chk = lay->check;
    if ((s = run_layout_check(lay, stream)) != MOC_OK) return s;
    return hip_status(moc_host::launch_varlen(lay, p, sel, nsel, counts, totals, tile_base, out,
                                              pair_count, static_cast<hipStream_t>(stream)),
                      "varlen launch");
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_build_varlen");
  }
}

// The guards of an attention call: the layout check (when moc_layout.check is set), then the
// capacity guard that writes vl->status, which every kernel of the call reads first.
static moc_status run_guards(const moc_layout* lay, const moc_varlen* vl, void* stream) {
  moc_status s = run_layout_check(lay, stream);
  if (s != MOC_OK) return s;
  return hip_status(moc_host::launch_varlen_guard(lay, vl, static_cast<hipStream_t>(stream)),
                    "varlen guard launch");
}

static moc_status check_varlen(const moc_layout* lay, const moc_varlen* vl) {
  if (!vl) return fail(MOC_EINVAL, "varlen is NULL");
  if (vl->S < 0 || vl->tile_rows != moc_host::attn_tile_rows() || !vl->bucket_off || !vl->bucket_q || !vl->slot ||
      !vl->rtiles || !vl->n_rtiles || !vl->atiles || !vl->n_atiles)
    return fail(MOC_EINVAL, "varlen struct not filled by moc_build_varlen");
  const VarlenSizes z = varlen_sizes(lay, vl->S);
  if (vl->max_rtiles != z.max_rtiles || vl->max_atiles != z.max_atiles ||
      vl->max_ktiles != z.max_ktiles || vl->n_text_split != z.n_text_split || !vl->ktiles ||
      !vl->n_ktiles || !vl->status || vl->routed_max != routed_max_of(lay, vl->S))
    return fail(MOC_EINVAL, "varlen struct built for another layout");
  if (vl->routed_cap < 0 || vl->routed_cap > vl->routed_max)
    return fail(MOC_EINVAL, "routed_cap %lld outside [0, %lld]",
                static_cast<long long>(vl->routed_cap), static_cast<long long>(vl->routed_max));
  return MOC_OK;
}

moc_status moc_attend_fwd(const moc_layout* lay, const moc_varlen* vl, const void* Q,
                          const void* K, const void* V, float softmax_scale, void* O, float* lse,
                          void* ws, size_t ws_bytes, void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    s = check_varlen(lay, vl);
    if (s != MOC_OK) return s;
    if (!Q || !K || !V || !O || !lse) return fail(MOC_EINVAL, "NULL tensor argument");
    if (O == Q || O == K || O == V || static_cast<const void*>(lse) == Q ||
        static_cast<const void*>(lse) == K || static_cast<const void*>(lse) == V)
      return fail(MOC_EINVAL, "outputs alias inputs");
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
      return fail(MOC_EINVAL, "softmax_scale must be finite and > 0");
    const size_t need = fwd_bytes(lay, vl->routed_cap);
    if (!ws || ws_bytes < need)
      return fail(MOC_EWORKSPACE, "FWD workspace needs %zu bytes (got %zu)", need,
                  ws ? ws_bytes : size_t(0));
    const int64_t rows = vl->routed_cap;
    char* w = static_cast<char*>(ws);
    float* pO = reinterpret_cast<float*>(w);
    w += align_up(sizeof(float) * (rows > 0 ? rows : 1) * lay->d);
    float* plse = reinterpret_cast<float*>(w);
    w += align_up(sizeof(float) * (rows > 0 ? rows : 1));
    void* vt = w;  // transposed V (bf16 layouts)
    if ((s = run_guards(lay, vl, stream)) != MOC_OK) return s;
    return hip_status(moc_host::launch_attn_fwd(lay, vl, Q, K, V, softmax_scale, O, lse, pO, plse,
                                                vt, static_cast<hipStream_t>(stream)),
                      "attention forward launch");
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_attend_fwd");
  }
}

moc_status moc_mx_quantize(const moc_layout* lay, const void* X, uint8_t* codes, uint8_t* scales,
                           void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    if (lay->dtype != MOC_BF16) return fail(MOC_EDTYPE, "MXFP8 quantisation takes bf16 input");
    if (!X || !codes || !scales) return fail(MOC_EINVAL, "NULL tensor argument");
    if (static_cast<const void*>(codes) == X || static_cast<const void*>(scales) == X ||
        codes == scales)
      return fail(MOC_EINVAL, "outputs alias");
    if ((s = run_layout_check(lay, stream)) != MOC_OK) return s;
    return hip_status(moc_host::launch_mx_quantize(lay, X, codes, scales,
                                                   static_cast<hipStream_t>(stream)),
                      "MXFP8 quantisation launch");
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_mx_quantize");
  }
}

moc_status moc_attend_fwd_mx(const moc_layout* lay, const moc_varlen* vl, const uint8_t* Qc,
                             const uint8_t* Qs, const uint8_t* Kc, const uint8_t* Ks,
                             const void* V, float softmax_scale, void* O, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    s = check_varlen(lay, vl);
    if (s != MOC_OK) return s;
    if (lay->dtype != MOC_BF16) return fail(MOC_EDTYPE, "quantised scores need a bf16 layout");
    if (!Qc || !Qs || !Kc || !Ks || !V || !O || !lse)
      return fail(MOC_EINVAL, "NULL tensor argument");
    const void* ins[] = {Qc, Qs, Kc, Ks, V};
    for (const void* a : ins)
      if (a == O || a == static_cast<const void*>(lse)) return fail(MOC_EINVAL, "outputs alias inputs");
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
      return fail(MOC_EINVAL, "softmax_scale must be finite and > 0");
    const size_t need = fwd_bytes(lay, vl->routed_cap);
    if (!ws || ws_bytes < need)
      return fail(MOC_EWORKSPACE, "FWD workspace needs %zu bytes (got %zu)", need,
                  ws ? ws_bytes : size_t(0));
    const int64_t rows = vl->routed_cap;
    char* w = static_cast<char*>(ws);
    float* pO = reinterpret_cast<float*>(w);
    w += align_up(sizeof(float) * (rows > 0 ? rows : 1) * lay->d);
    float* plse = reinterpret_cast<float*>(w);
    w += align_up(sizeof(float) * (rows > 0 ? rows : 1));
    if ((s = run_guards(lay, vl, stream)) != MOC_OK) return s;
    return hip_status(moc_host::launch_attn_fwd_mx(lay, vl, Qc, Qs, Kc, Ks, V, softmax_scale, O,
                                                   lse, pO, plse, w,
                                                   static_cast<hipStream_t>(stream)),
                      "quantised-scores attention forward launch");
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_attend_fwd_mx");
  }
}

size_t moc_mx_quantize_v_bytes(const moc_layout* lay) {
  try {
    if (check_layout(lay) != MOC_OK) return 0;
    if (lay->dtype != MOC_BF16) {
      fail(MOC_EDTYPE, "MXFP8 quantisation takes bf16 input");
      return 0;
    }
    return moc_host::mx_quantize_v_bytes(lay);
  } catch (...) {
    fail(MOC_EINTERNAL, "exception in moc_mx_quantize_v_bytes");
    return 0;
  }
}

moc_status moc_mx_quantize_v(const moc_layout* lay, const void* V, uint8_t* vq, void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    if (lay->dtype != MOC_BF16) return fail(MOC_EDTYPE, "MXFP8 quantisation takes bf16 input");
    if (!V || !vq) return fail(MOC_EINVAL, "NULL tensor argument");
    if (static_cast<const void*>(vq) == V) return fail(MOC_EINVAL, "output aliases the input");
    if ((s = run_layout_check(lay, stream)) != MOC_OK) return s;
    return hip_status(moc_host::launch_mx_quantize_v(lay, V, vq, static_cast<hipStream_t>(stream)),
                      "MXFP8 value quantisation launch");
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_mx_quantize_v");
  }
}

moc_status moc_attend_fwd_mxv(const moc_layout* lay, const moc_varlen* vl, const uint8_t* Qc,
                              const uint8_t* Qs, const uint8_t* Kc, const uint8_t* Ks,
                              const uint8_t* Vq, float softmax_scale, void* O, float* lse,
                              void* ws, size_t ws_bytes, void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    s = check_varlen(lay, vl);
    if (s != MOC_OK) return s;
    if (lay->dtype != MOC_BF16) return fail(MOC_EDTYPE, "quantised values need a bf16 layout");
    if (!Qc || !Qs || !Kc || !Ks || !Vq || !O || !lse)
      return fail(MOC_EINVAL, "NULL tensor argument");
    const void* ins[] = {Qc, Qs, Kc, Ks, Vq};
    for (const void* a : ins)
      if (a == O || a == static_cast<const void*>(lse)) return fail(MOC_EINVAL, "outputs alias inputs");
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
      return fail(MOC_EINVAL, "softmax_scale must be finite and > 0");
    const size_t need = fwd_bytes(lay, vl->routed_cap);
    if (!ws || ws_bytes < need)
      return fail(MOC_EWORKSPACE, "FWD workspace needs %zu bytes (got %zu)", need,
                  ws ? ws_bytes : size_t(0));
    const int64_t rows = vl->routed_cap;
    char* w = static_cast<char*>(ws);
    float* pO = reinterpret_cast<float*>(w);
    w += align_up(sizeof(float) * (rows > 0 ? rows : 1) * lay->d);
    float* plse = reinterpret_cast<float*>(w);
    if ((s = run_guards(lay, vl, stream)) != MOC_OK) return s;
    return hip_status(moc_host::launch_attn_fwd_mxv(lay, vl, Qc, Qs, Kc, Ks, Vq, softmax_scale, O,
                                                    lse, pO, plse,
                                                    static_cast<hipStream_t>(stream)),
                      "quantised-values attention forward launch");
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_attend_fwd_mxv");
  }
}

moc_status moc_attend_bwd(const moc_layout* lay, const moc_varlen* vl, const void* Q,
                          const void* K, const void* V, const void* O, const float* lse,
                          const void* dO, float softmax_scale, void* dQ, void* dK, void* dV,
                          void* ws, size_t ws_bytes, void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    s = check_varlen(lay, vl);
    if (s != MOC_OK) return s;
    if (!Q || !K || !V || !O || !lse || !dO || !dQ || !dK || !dV)
      return fail(MOC_EINVAL, "NULL tensor argument");
    const void* ins[] = {Q, K, V, O, lse, dO};
    const void* outs[] = {dQ, dK, dV};
    for (const void* a : outs)
      for (const void* b : ins)
        if (a == b) return fail(MOC_EINVAL, "outputs alias inputs");
    if (dQ == dK || dQ == dV || dK == dV) return fail(MOC_EINVAL, "gradient outputs alias");
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
      return fail(MOC_EINVAL, "softmax_scale must be finite and > 0");
    const size_t need = moc_host::attn_bwd_workspace(lay, vl->routed_cap);
    if (!ws || ws_bytes < need)
      return fail(MOC_EWORKSPACE, "BWD workspace needs %zu bytes (got %zu)", need,
                  ws ? ws_bytes : size_t(0));
    if (lay->dtype != MOC_BF16) return fail(MOC_EUNSUPPORTED, "backward not available");
    if ((s = run_guards(lay, vl, stream)) != MOC_OK) return s;
    hipError_t e = moc_host::launch_attn_bwd(lay, vl, Q, K, V, O, lse, dO, softmax_scale, dQ, dK,
                                             dV, ws, ws_bytes, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return fail(MOC_EUNSUPPORTED, "backward not available");
    return hip_status(e, "attention backward launch");
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_attend_bwd");
  }
}

moc_status moc_check_layout(const moc_layout* lay, void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    if (!lay->check) return fail(MOC_EINVAL, "moc_check_layout needs lay->check");
    return run_layout_check(lay, stream);
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_check_layout");
  }
}

uint32_t moc_layout_check_host(const int32_t* chunk_offsets, const int32_t* chunk_shot, int32_t C,
                               int32_t L, int32_t text_begin, int32_t text_end) {
  if (!chunk_offsets || !chunk_shot || C < 1) return MOC_LAYOUT_BAD_START | MOC_LAYOUT_BAD_END;
  return moc_host::layout_check_host(chunk_offsets, chunk_shot, C, L, text_begin, text_end);
}

moc_status moc_layout_status(uint32_t word) {
  if (word == 0) return MOC_OK;
  static const struct { uint32_t bit; const char* what; } kBits[] = {
      {MOC_LAYOUT_BAD_START, "chunk_offsets[0] != 0"},
      {MOC_LAYOUT_NOT_INCREASING, "chunk offsets not strictly increasing"},
      {MOC_LAYOUT_BAD_END, "chunk_offsets[C] != L"},
      {MOC_LAYOUT_BAD_SHOT_ID, "a shot id below -1"},
      {MOC_LAYOUT_BAD_TEXT, "a chunk straddles the text range, or shot -1 is not exactly the "
                            "text chunks"},
      {MOC_LAYOUT_SHOT_SPLIT, "a shot's chunks are not contiguous"},
  };
  std::string msg = "layout check word 0x";
  char hex[16];
  snprintf(hex, sizeof(hex), "%x", word);
  msg += hex;
  for (const auto& b : kBits)
    if (word & b.bit) msg += std::string("; ") + b.what;
  return fail(MOC_ELAYOUT, "%s", msg.c_str());
}

moc_status moc_varlen_total(const moc_layout* lay, const moc_varlen* vl, int64_t* total,
                            void* stream) {
  try {
    moc_status s = check_layout(lay);
    if (s != MOC_OK) return s;
    if ((s = check_varlen(lay, vl)) != MOC_OK) return s;
    if (!total) return fail(MOC_EINVAL, "total is NULL");
    s = hip_status(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "stream synchronise");
    if (s != MOC_OK) return s;
    if (lay->check) {
      // a rejected layout left the inversion unwritten: there is no total to report
      uint32_t word = 0;
      s = hip_status(hipMemcpy(&word, lay->check, sizeof(word), hipMemcpyDeviceToHost),
                     "copy of the layout check word");
      if (s != MOC_OK) return s;
      if (word != 0) return moc_layout_status(word);
    }
    const int64_t nb = static_cast<int64_t>(lay->B) * lay->H * lay->C;
    int32_t v = 0;
    s = hip_status(hipMemcpy(&v, vl->bucket_off + nb, sizeof(v), hipMemcpyDeviceToHost),
                   "copy of the routed total");
    if (s != MOC_OK) return s;
    *total = v;
    return MOC_OK;
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_varlen_total");
  }
}

moc_status moc_varlen_set_capacity(moc_varlen* vl, int64_t routed_cap) {
  if (!vl || !vl->status) return fail(MOC_EINVAL, "varlen struct not filled by moc_build_varlen");
  if (routed_cap < 0 || routed_cap > vl->routed_max)
    return fail(MOC_EINVAL, "routed_cap %lld outside [0, %lld]",
                static_cast<long long>(routed_cap), static_cast<long long>(vl->routed_max));
  vl->routed_cap = routed_cap;
  return MOC_OK;
}

size_t moc_attend_workspace_bytes(const moc_layout* lay, const moc_varlen* vl, int32_t op) {
  if (check_layout(lay) != MOC_OK) return 0;
  if (check_varlen(lay, vl) != MOC_OK) return 0;
  if (op == MOC_OP_FWD) return fwd_bytes(lay, vl->routed_cap);
  if (op == MOC_OP_BWD) return moc_host::attn_bwd_workspace(lay, vl->routed_cap);
  fail(MOC_EINVAL, "op must be MOC_OP_FWD or MOC_OP_BWD (got %d)", op);
  return 0;
}

moc_status moc_varlen_status(const moc_varlen* vl, void* stream) {
  try {
    if (!vl || !vl->status) return fail(MOC_EINVAL, "varlen struct not filled by moc_build_varlen");
    moc_status s = hip_status(hipStreamSynchronize(static_cast<hipStream_t>(stream)),
                              "stream synchronise");
    if (s != MOC_OK) return s;
    uint32_t w = 0;
    s = hip_status(hipMemcpy(&w, vl->status, sizeof(w), hipMemcpyDeviceToHost),
                   "copy of the status word");
    if (s != MOC_OK) return s;
    if (w & MOC_VARLEN_OVER_CAPACITY)
      return fail(MOC_EWORKSPACE, "the routing has more routed rows than routed_cap = %lld; the "
                                  "attention call wrote nothing",
                  static_cast<long long>(vl->routed_cap));
    if (w & MOC_VARLEN_BAD_LAYOUT)
      return fail(MOC_ELAYOUT, "the layout check word was set; the attention call wrote nothing");
    return MOC_OK;
  } catch (...) {
    return fail(MOC_EINTERNAL, "exception in moc_varlen_status");
  }
}

}  // extern "C"
