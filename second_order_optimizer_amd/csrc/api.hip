// The extern "C" entry points of include/kfac.h: host-side validation,
// workspace sizing and dispatch to the diagonal and full launchers.
#include "common.h"

#include <algorithm>
#include <cmath>
#include <cstring>

namespace kfac {

LayerGeom geom_of(const kfac_layer_t& L) {
  LayerGeom g{};
  g.rows = L.rows;
  g.d_in = L.d_in;
  g.d_out = L.d_out;
  g.bias = L.has_bias != 0;
  g.d_a = L.d_in + (g.bias ? 1 : 0);
  g.conv = L.kind == KFAC_CONV2D;
  g.bn = L.kind == KFAC_BATCHNORM;
  g.packed = L.factor_layout == KFAC_FACTORS_PACKED;
  if (g.conv || g.bn) {
    g.batch = L.batch;
    g.c_in = L.c_in;
    g.h = L.height;
    g.w = L.width;
    g.kh = L.kh;
    g.kw = L.kw;
    g.stride = L.stride;
    g.pad = L.pad;
    g.h_out = L.stride > 0 ? (L.height + 2 * L.pad - L.kh) / L.stride + 1 : 0;
    g.w_out = L.stride > 0 ? (L.width + 2 * L.pad - L.kw) / L.stride + 1 : 0;
  }
  return g;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape / dtype checks that do not look at pointers.
kfac_status_t check_shape(const kfac_layer_t& L, int mode) {
  if (L.kind != KFAC_LINEAR && L.kind != KFAC_CONV2D && L.kind != KFAC_BATCHNORM) return KFAC_ERR_ARG;
  if (L.has_bias != 0 && L.has_bias != 1) return KFAC_ERR_ARG;
  if (L.reserved != 0) return KFAC_ERR_ARG;
  if (L.factor_layout != KFAC_FACTORS_FULL && L.factor_layout != KFAC_FACTORS_PACKED) return KFAC_ERR_ARG;
  if (L.act_dtype != KFAC_F32 && L.act_dtype != KFAC_BF16) return KFAC_ERR_DTYPE;
  if (L.grad_dtype != KFAC_F32 && L.grad_dtype != KFAC_BF16) return KFAC_ERR_DTYPE;
  if (L.d_in <= 0 || L.d_out <= 0 || L.rows <= 0) return KFAC_ERR_ARG;
  // int32 element indexing of parameter matrices and of per-sample planes
  if (static_cast<int64_t>(L.d_out) * (L.d_in + 1) >= (int64_t(1) << 31)) return KFAC_ERR_UNSUPPORTED;
  if (L.kind == KFAC_BATCHNORM) {
    // gamma, beta over C planes of height x width per sample
    if (L.batch <= 0 || L.c_in <= 0 || L.height <= 0 || L.width <= 0) return KFAC_ERR_ARG;
    if (L.d_in != 1 || L.d_out != L.c_in || L.rows != L.batch) return KFAC_ERR_ARG;
    if (L.kh != 1 || L.kw != 1 || L.stride != 1 || L.pad != 0) return KFAC_ERR_ARG;
    if (L.act_dtype != KFAC_F32 || L.grad_dtype != KFAC_F32) return KFAC_ERR_DTYPE;
    if (static_cast<int64_t>(L.c_in) * L.height * L.width >= (int64_t(1) << 31)) return KFAC_ERR_UNSUPPORTED;
    return KFAC_OK;
  }
  if (L.kind == KFAC_CONV2D) {
    if (L.batch <= 0 || L.c_in <= 0 || L.height <= 0 || L.width <= 0 || L.kh <= 0 || L.kw <= 0 || L.stride <= 0 ||
        L.pad < 0)
      return KFAC_ERR_ARG;
    if (L.kh != L.kw || L.kh > 7) return KFAC_ERR_UNSUPPORTED;
    // convolution inputs and gradients are read as float32
    if (L.act_dtype != KFAC_F32 || L.grad_dtype != KFAC_F32) return KFAC_ERR_DTYPE;
    const int64_t ho = (static_cast<int64_t>(L.height) + 2 * L.pad - L.kh) / L.stride + 1;
    const int64_t wo = (static_cast<int64_t>(L.width) + 2 * L.pad - L.kw) / L.stride + 1;
    if (L.height + 2 * L.pad < L.kh || L.width + 2 * L.pad < L.kw || ho <= 0 || wo <= 0) return KFAC_ERR_ARG;
    if (static_cast<int64_t>(L.c_in) * L.kh * L.kw != L.d_in) return KFAC_ERR_ARG;
    if (static_cast<int64_t>(L.batch) * ho * wo != L.rows) return KFAC_ERR_ARG;
    if (static_cast<int64_t>(L.c_in) * L.height * L.width >= (int64_t(1) << 31)) return KFAC_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(L.d_out) * ho * wo >= (int64_t(1) << 31)) return KFAC_ERR_UNSUPPORTED;
  }
  if (mode == KFAC_MODE_DIAG) {
    // the diagonal reduction streams float32 inputs
    if (L.act_dtype != KFAC_F32 || L.grad_dtype != KFAC_F32) return KFAC_ERR_DTYPE;
  }
  if (mode == KFAC_MODE_FULL) {
    // the fp32 factor contractions (and the conv row layout) count rows in
    // 32 bits; bf16 factors are split into row chunks and have no such limit
    const bool fp32_rows = L.kind == KFAC_CONV2D || L.act_dtype == KFAC_F32 || L.grad_dtype == KFAC_F32;
    if (fp32_rows && L.rows > INT32_MAX) return KFAC_ERR_UNSUPPORTED;
  }
  return KFAC_OK;
}

kfac_status_t check_ptr(const void* p, bool required) {
  if (!p) return required ? KFAC_ERR_ARG : KFAC_OK;
  return aligned16(p) ? KFAC_OK : KFAC_ERR_ALIGN;
}

kfac_status_t check_layer_ptrs(const kfac_layer_t& L, int mode, int phases, int refresh, int options) {
  const bool bias = L.has_bias != 0;
  kfac_status_t s;
  auto req = [&](const void* p, bool r) { return (s = check_ptr(p, r)) != KFAC_OK; };
  const bool fac = phases & KFAC_PHASE_FACTORS;
  const bool upd = phases & KFAC_PHASE_UPDATE;
  const bool inv = (phases & KFAC_PHASE_INVERT) && refresh != 0;
  if (req(L.a, fac) || req(L.g, fac)) return s;
  // the weight rescaling writes the weight of every conv / linear layer
  const bool resc = (phases & KFAC_PHASE_RESCALE) && (options & KFAC_OPT_RESCALE) && L.kind != KFAC_BATCHNORM;
  if (req(L.grad_w, upd) || req(L.w, upd || resc) || req(L.mom_w, upd)) return s;
  if (bias && (req(L.grad_b, upd) || req(L.b, upd) || req(L.mom_b, upd))) return s;
  if (!bias && (L.grad_b || L.b || L.mom_b || L.F_b)) return KFAC_ERR_ARG;
  if (mode == KFAC_MODE_FULL && L.kind != KFAC_BATCHNORM) {
    if (req(L.A, fac || inv) || req(L.G, fac || inv)) return s;
    if (req(L.A_inv, inv || upd) || req(L.G_inv, inv || upd)) return s;
  } else {
    if (req(L.dA, fac || upd) || req(L.dG, fac || upd)) return s;
    if (req(L.F_w, upd)) return s;
    if (bias && req(L.F_b, upd)) return s;
  }
  return KFAC_OK;
}

kfac_status_t check_all(const kfac_layer_t* layers, int32_t n, int mode) {
  if (!layers || n <= 0) return KFAC_ERR_ARG;
  for (int i = 0; i < n; ++i) {
    kfac_status_t s = check_shape(layers[i], mode);
    if (s != KFAC_OK) return s;
  }
  return KFAC_OK;
}

// Descriptor, scalar and pointer checks shared by the step entry points;
// *phases receives the phases the call runs.
kfac_status_t validate(const kfac_layer_t* layers, int32_t n, const kfac_hparams_t* hp, int mode, int* phases) {
  kfac_status_t s = check_all(layers, n, mode);
  if (s != KFAC_OK) return s;
  if (!hp || hp->reserved != 0) return KFAC_ERR_ARG;
  if (hp->phase_mask < 0 || hp->phase_mask > KFAC_PHASE_ALL) return KFAC_ERR_ARG;
  if (hp->refresh < 0 || hp->refresh > KFAC_REFRESH_BOTH) return KFAC_ERR_ARG;
  if ((hp->options & ~KFAC_OPT_RESCALE) != 0) return KFAC_ERR_ARG;
  *phases = hp->phase_mask == 0 ? KFAC_PHASE_ALL : hp->phase_mask;
  for (int i = 0; i < n; ++i) {
    s = check_layer_ptrs(layers[i], mode, *phases, hp->refresh, hp->options);
    if (s != KFAC_OK) return s;
  }
  return KFAC_OK;
}

kfac_status_t run(const kfac_layer_t* layers, int32_t n, const kfac_hparams_t* hp, void* workspace,
                  size_t ws_bytes, void* stream, int mode) {
  int phases = 0;
  kfac_status_t s = validate(layers, n, hp, mode, &phases);
  if (s != KFAC_OK) return s;
  if (!workspace) return KFAC_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KFAC_ERR_ALIGN;
  const size_t need = mode == KFAC_MODE_FULL ? full_workspace_bytes(layers, n) : diag_workspace_bytes(layers, n);
  if (ws_bytes < need) return KFAC_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (mode == KFAC_MODE_FULL) return full_enqueue(layers, n, *hp, ws, ws_bytes, st, phases);
  return diag_enqueue(layers, n, *hp, ws, ws_bytes, st, phases);
}

}  // namespace
}  // namespace kfac

extern "C" {

kfac_status_t kfac_workspace_size(const kfac_layer_t* layers, int32_t n_layers, int32_t mode, size_t* bytes) {
  if (!bytes) return KFAC_ERR_ARG;
  if (mode != KFAC_MODE_FULL && mode != KFAC_MODE_DIAG) return KFAC_ERR_ARG;
  kfac_status_t s = kfac::check_all(layers, n_layers, mode);
  if (s != KFAC_OK) return s;
  *bytes = mode == KFAC_MODE_FULL ? kfac::full_workspace_bytes(layers, n_layers)
                                  : kfac::diag_workspace_bytes(layers, n_layers);
  return KFAC_OK;
}

kfac_status_t kfac_step_full(const kfac_layer_t* layers, int32_t n_layers, const kfac_hparams_t* hp,
                             void* workspace, size_t ws_bytes, void* stream) {
  return kfac::run(layers, n_layers, hp, workspace, ws_bytes, stream, KFAC_MODE_FULL);
}

kfac_status_t kfac_step_diag(const kfac_layer_t* layers, int32_t n_layers, const kfac_hparams_t* hp,
                             void* workspace, size_t ws_bytes, void* stream) {
  return kfac::run(layers, n_layers, hp, workspace, ws_bytes, stream, KFAC_MODE_DIAG);
}

kfac_status_t kfac_step_diag_noalloc(const kfac_layer_t* layers, int32_t n_layers, const kfac_hparams_t* hp,
                                     uint32_t* flags, void* stream) {
  int phases = 0;
  kfac_status_t s = kfac::validate(layers, n_layers, hp, KFAC_MODE_DIAG, &phases);
  if (s != KFAC_OK) return s;
  if (!flags) return KFAC_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(flags) & 3u) != 0) return KFAC_ERR_ALIGN;
  return kfac::diag_enqueue_noalloc(layers, n_layers, *hp, flags, static_cast<hipStream_t>(stream), phases);
}

kfac_status_t kfac_read_flags(void* workspace, void* stream, uint32_t* flags, int32_t clear) {
  if (!workspace || !flags) return KFAC_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t h = 0;
  if (hipMemcpyAsync(&h, workspace, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess) return KFAC_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return KFAC_ERR_HIP;
  *flags = h;
  if (clear) {
    if (hipMemsetAsync(workspace, 0, sizeof(uint32_t), st) != hipSuccess) return KFAC_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return KFAC_ERR_HIP;
  }
  return KFAC_OK;
}

kfac_status_t kfac_schedule_hparams(const kfac_schedule_t* sc, int64_t step, kfac_hparams_t* hp) {
  if (!sc || !hp || step < 1) return KFAC_ERR_ARG;
  if (sc->warmup_steps < 0 || sc->dense_steps < 0 || sc->refresh_every_a < 1 || sc->refresh_every_g < 1)
    return KFAC_ERR_ARG;
  if (sc->warmup_shape != KFAC_WARMUP_LINEAR && sc->warmup_shape != KFAC_WARMUP_GEOMETRIC) return KFAC_ERR_ARG;
  const double g0 = sc->damping_init, gt = sc->damping_target;
  if (sc->warmup_shape == KFAC_WARMUP_GEOMETRIC && !(g0 > 0.0 && gt > 0.0)) return KFAC_ERR_ARG;
  // warm-up damping: fraction u of the way from the initial to the target value
  const double u = sc->warmup_steps == 0
                       ? 1.0
                       : static_cast<double>(std::min<int64_t>(step - 1, sc->warmup_steps)) / sc->warmup_steps;
  const double lam = sc->warmup_shape == KFAC_WARMUP_LINEAR ? g0 + (gt - g0) * u : g0 * std::pow(gt / g0, u);
  hp->damping = static_cast<float>(lam);
  hp->damping_bn = static_cast<float>(static_cast<double>(sc->bn_damping_scale) * lam);
  // refresh: every step up to D, then each factor on its own interval
  const int64_t D = std::max<int64_t>(sc->dense_steps, 1);
  const bool ra = step <= D || (step - D) % sc->refresh_every_a == 0;
  const bool rg = step <= D || (step - D) % sc->refresh_every_g == 0;
  hp->refresh = (ra ? KFAC_REFRESH_A : 0) | (rg ? KFAC_REFRESH_G : 0);
  return KFAC_OK;
}

const char* kfac_status_string(kfac_status_t s) {
  switch (s) {
    case KFAC_OK: return "ok";
    case KFAC_ERR_ARG: return "invalid argument";
    case KFAC_ERR_DTYPE: return "unsupported dtype for this operand";
    case KFAC_ERR_ALIGN: return "misaligned pointer";
    case KFAC_ERR_WORKSPACE: return "workspace missing or too small";
    case KFAC_ERR_UNSUPPORTED: return "unsupported layer configuration";
    case KFAC_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t kfac_abi_version(void) { return KFAC_ABI_VERSION; }

}  // extern "C"
