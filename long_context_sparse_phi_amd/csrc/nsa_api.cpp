// C ABI of the NSA library: argument validation, workspace layout and the
// launch sequence of each entry point.  Nothing is enqueued until every check
// has passed.
#include <hip/hip_runtime.h>

#include <atomic>
#include <initializer_list>
#include <cmath>
#include <cstring>

#include "../../include/nsa.h"
#include "nsa_kernels.hpp"

namespace nsa {
constexpr int kPrefillStages = 8;
constexpr int kDecodeStages = 3;
int bwd_stage_count();
bool cmp_out_fits(const Dims& dm);
hipError_t launch_decode(const Dims& dm, const nsa_decode_args* a, void* ws, hipStream_t s,
                         void* const* events);
size_t decode_ws_bytes(const Dims& dm);
bool decode_fits(const Dims& dm);
hipError_t decode_static_scratch(void** out);
hipError_t launch_bwd(const Dims& dm, const nsa_bwd_args* a, void* ws, hipStream_t s, void* const* events);
size_t bwd_ws_bytes(const Dims& dm);
size_t dense_bwd_ws_bytes(const Dims& dm);
bool dense_bwd_supported(const Dims& dm);
hipError_t launch_dense_bwd(const Dims& dm, const nsa_dense_bwd_args* a, void* ws, hipStream_t s);
}  // namespace nsa

using namespace nsa;

namespace {

constexpr size_t kAlign = 256;
inline size_t al(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Bump allocator over the caller's workspace.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += al(bytes);
    return p;
  }
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Device check: gfx950 only.  Cached per device id; the cache holds no state
// that changes results.
nsa_status check_device() {
  static std::atomic<int> ok[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NSA_ERR_HIP;
  if (dev < 0 || dev >= 64) return NSA_ERR_UNSUPPORTED;
  int v = ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NSA_ERR_HIP;
    v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? NSA_OK : NSA_ERR_UNSUPPORTED;
}

// Validates p and fills the derived sizes.  T_override: sequence length to
// use (the cache length for decode).
nsa_status make_dims(const nsa_params* p, Dims* dm) {
  if (!p || !dm) return NSA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->seqlen < 1 || p->n_kv_heads < 1 || p->group_size < 1) return NSA_ERR_INVALID_ARG;
  const int G = p->group_size;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return NSA_ERR_UNSUPPORTED;
  if (p->d_k < 1 || p->d_v < 1) return NSA_ERR_INVALID_ARG;
  if (!shapes_supported(p->d_k, p->d_v)) return NSA_ERR_UNSUPPORTED;
  // one key row of every KV head: a 24-bit element count (decode tile addressing)
  if ((long long)p->n_kv_heads * (p->d_k > p->d_v ? p->d_k : p->d_v) >= (1ll << 24)) return NSA_ERR_UNSUPPORTED;
  const int l = p->cmp_block, d = p->cmp_stride, ls = p->sel_block;
  if (l < 1 || d < 1 || ls < 1 || l % d != 0 || ls % d != 0 || l > ls) return NSA_ERR_INVALID_ARG;
  if (ls % 16 != 0 || (32 * d) % ls != 0) return NSA_ERR_UNSUPPORTED;
  if ((31 * d + l - 1) / ls + 1 > 32) return NSA_ERR_UNSUPPORTED;
  if (p->n_select < 3 || p->n_select > 32) return NSA_ERR_INVALID_ARG;
  if (p->window < 1) return NSA_ERR_INVALID_ARG;
  if (p->gate_dim < 1) return NSA_ERR_INVALID_ARG;
  if (p->gate_dim > 1024) return NSA_ERR_UNSUPPORTED;
  if (p->gate_hidden < 0 || p->gate_hidden > 1024) return NSA_ERR_INVALID_ARG;
  if (p->phi != NSA_PHI_MEANPOOL && p->phi != NSA_PHI_MLP) return NSA_ERR_INVALID_ARG;
  if (p->phi == NSA_PHI_MLP && (p->phi_hidden < 64 || p->phi_hidden % 64 != 0)) return NSA_ERR_INVALID_ARG;
  if (p->io_dtype != NSA_BF16 && p->io_dtype != NSA_FP32) return NSA_ERR_UNSUPPORTED;
  if (!(p->scale >= 0.f) || std::isinf(p->scale)) return NSA_ERR_INVALID_ARG;
  const long long tokens = (long long)p->batch * p->seqlen * p->n_kv_heads * G;
  if (tokens * (p->d_k > p->d_v ? p->d_k : p->d_v) >= (1ll << 40)) return NSA_ERR_UNSUPPORTED;
  Dims& D = *dm;
  D.B = p->batch; D.T = p->seqlen; D.Hkv = p->n_kv_heads; D.G = G; D.Hq = p->n_kv_heads * G;
  D.dk = p->d_k; D.dv = p->d_v; D.l = l; D.d = d; D.ls = ls; D.n = p->n_select; D.w = p->window;
  D.ncmp = D.T < l ? 0 : (D.T - l) / d + 1;
  D.ncmp_pad = ((D.ncmp + 63) & ~63) + 64;
  D.nsel = (D.T + ls - 1) / ls;
  D.Tp = ((D.T + 63) & ~63) + 64;
  D.C = p->gate_dim;
  D.Cg = p->gate_hidden;
  D.hidden = p->phi == NSA_PHI_MLP ? p->phi_hidden : 0;
  D.scale = p->scale > 0.f ? p->scale : 1.f / std::sqrt((float)p->d_k);
  D.io = p->io_dtype == NSA_BF16 ? IO_BF16 : IO_F32;
  if (!cmp_out_fits(D)) return NSA_ERR_UNSUPPORTED;
  return NSA_OK;
}

size_t esize(const Dims& dm) { return dm.io == IO_BF16 ? 2 : 4; }

// Workspace plan of the prefill forward.  Every optional output the caller
// leaves NULL is placed in the workspace; sizes assume all are NULL.
struct PrefillWs {
  void *gates, *gh, *kc, *vc, *vct, *vt, *kvf, *lse, *idx, *ob, *phi;
};

size_t phi_ws(const Dims& dm) {
  if (dm.hidden == 0) return 0;
  size_t a = phi_mlp_ws_bytes(dm, dm.dk), b = phi_mlp_ws_bytes(dm, dm.dv);
  return a > b ? a : b;
}

size_t plan_prefill(const Dims& dm, void* ws, PrefillWs* w) {
  Carve c(ws);
  const size_t BTH = (size_t)dm.B * dm.T * dm.Hq;
  const size_t es = esize(dm);
  w->gates = c.take(BTH * 3 * 4);
  w->gh = c.take((size_t)dm.B * dm.T * dm.Cg * 4);
  w->kc = c.take((size_t)dm.B * dm.ncmp * dm.Hkv * dm.dk * es);
  w->vc = c.take((size_t)dm.B * dm.ncmp * dm.Hkv * dm.dv * es);
  w->vct = c.take((size_t)dm.B * dm.Hkv * dm.dv * dm.ncmp_pad * es);
  w->vt = c.take((size_t)dm.B * dm.Hkv * dm.dv * dm.Tp * es);
  w->kvf = c.take(kv_frag_elems(dm) * es);
  w->lse = c.take(3 * BTH * 4);
  w->idx = c.take((size_t)dm.B * dm.T * dm.Hkv * dm.n * 4);
  w->ob = c.take(2 * BTH * dm.dv * es);
  w->phi = c.take(phi_ws(dm));
  return c.off;
}

nsa_status hip_status(hipError_t e) { return e == hipSuccess ? NSA_OK : NSA_ERR_HIP; }

// Dense baseline workspace: the transposed V the window kernel reads.
size_t dense_ws_bytes(const Dims& dm) { return (size_t)dm.B * dm.Hkv * dm.dv * dm.Tp * esize(dm) + 256; }

// Compress one tensor (keys: D = dk, values: D = dv) into out (and outT).
hipError_t run_compress(const Dims& dm, int D, const void* x, const nsa_phi_weights* phi, void* out,
                        void* outT, void* phi_ws_ptr, hipStream_t s) {
  if (dm.hidden == 0) return launch_meanpool(dm, D, x, out, outT, s);
  PhiMlpArgs a;
  a.D = D; a.x = x; a.pe = phi->pe; a.w1 = phi->w1; a.b1 = phi->b1; a.w2 = phi->w2; a.b2 = phi->b2;
  Carve c(phi_ws_ptr);
  const size_t es = esize(dm);
  const int R = dm.l / dm.d;
  const int nsub = dm.ncmp > 0 ? dm.ncmp + R - 1 : 0;
  a.arows = c.take(((size_t)dm.B * dm.Hkv * nsub + R) * dm.d * D * es);
  a.w2t = c.take((size_t)D * dm.hidden * es);
  a.pe_part = (float*)c.take(phi_pe_part_floats(dm) * 4);
  a.y = (float*)c.take(((size_t)dm.B * dm.Hkv * nsub + R) * R * dm.hidden * 4);
  a.h = c.take((size_t)dm.B * dm.Hkv * dm.ncmp * dm.hidden * 4);
  a.out = out; a.outT = outT;
  return launch_phi_mlp(dm, a, s);
}

// Records caller-provided events between stages (no-op without events).
struct Stages {
  void* const* ev;
  hipStream_t s;
  int i = 0;
  Stages(void* const* e, hipStream_t st) : ev(e), s(st) {}
  // true on failure
  bool mark() { return ev ? hipEventRecord((hipEvent_t)ev[i++], s) != hipSuccess : false; }
};

// The optional per-branch tensors are either all absent or all present and aligned.
bool all_or_none(std::initializer_list<const void*> ps, bool* present) {
  int n = 0, k = 0;
  for (const void* p : ps) {
    ++k;
    if (p) {
      if (!aligned16(p)) return false;
      ++n;
    }
  }
  *present = n > 0;
  return n == 0 || n == k;
}

// Gate MLP weights: required (aligned) when the gate has a hidden layer.
bool gate_ok(const Dims& dm, const nsa_gate_mlp& g) {
  if (dm.Cg == 0) return true;
  const void* ps[3] = {g.w1, g.b1, g.b2};
  for (const void* p : ps)
    if (!p || !aligned16(p)) return false;
  return true;
}

bool phi_ok(const nsa_phi_weights& w) {
  const void* ps[5] = {w.pe, w.w1, w.b1, w.w2, w.b2};
  for (const void* p : ps)
    if (!p || !aligned16(p)) return false;
  return true;
}

// ---------------------------------------------------------------------------
// Projection layer: hand-written GEMMs (nsa_gemm.hip) around the operator.
// ---------------------------------------------------------------------------

// split-K bound of the layer's weight-gradient GEMMs (sums over every token)
constexpr int kLayerSplit = 8;

struct LayerBwdWs {
  void* op_ws;    // the operator's backward workspace
  void* d_o;      // dO = dy w_o^T, io dtype [B*T, Hq*dv]
  float *dq, *dk, *dv;
  float* part;    // split-K partials of the weight gradients
};

size_t plan_layer_bwd(const Dims& dm, void* ws, LayerBwdWs* w) {
  Carve c(ws);
  LayerBwdWs t;
  if (!w) w = &t;
  const size_t ntok = (size_t)dm.B * dm.T, es = esize(dm);
  w->op_ws = c.take(bwd_ws_bytes(dm));
  w->d_o = c.take(ntok * dm.Hq * dm.dv * es);
  w->dq = (float*)c.take(ntok * dm.Hq * dm.dk * 4);
  w->dk = (float*)c.take(ntok * dm.Hkv * dm.dk * 4);
  w->dv = (float*)c.take(ntok * dm.Hkv * dm.dv * 4);
  // partials of dW_o [Hq*dv, C] or of dW_q|dW_k|dW_v [C, Hq*dk + Hkv*(dk + dv)]
  const size_t nqkv = (size_t)dm.Hq * dm.dk + (size_t)dm.Hkv * (dm.dk + dm.dv);
  const size_t wmax = (size_t)dm.C * (nqkv > (size_t)dm.Hq * dm.dv ? nqkv : (size_t)dm.Hq * dm.dv);
  w->part = (float*)c.take(wmax * (dm.io == IO_BF16 ? kLayerSplit : kGemmMaxSplit) * 4);
  return c.off;
}

// One layer GEMM: C = A B (+ C), bf16 MFMA for bf16 I/O (fp32 operands as
// hi + lo parts), exact fp32 MFMA for fp32 I/O.  a_f32 / b_f32: the operand is
// fp32 whatever the I/O type.  split: the sum runs over many tokens.
hipError_t layer_gemm(const Dims& dm, const MmArgs& g, bool a_f32, bool b_f32, bool split, float* part,
                      hipStream_t s) {
  if (dm.io == IO_BF16) return mm(g, a_f32, b_f32, split ? mm_split(g, kLayerSplit) : 1, part, s);
  const Gemm e{g.M, g.N, g.K, g.A, g.sam, g.sak, g.B, g.sbk, g.sbn, (float*)g.C, g.ldc, g.accumulate};
  return gemm_exact(e, true, true, split ? part : nullptr, s);
}

// The q|k|v products of the layer as one launch over three segments (see
// MmArgs).  With fp32 I/O the exact fp32 GEMM runs once per segment.
hipError_t layer_gemm_seg(const Dims& dm, const MmArgs& g, bool a_f32, bool b_f32, bool split, float* part,
                          hipStream_t s) {
  if (dm.io == IO_BF16) return mm(g, a_f32, b_f32, split ? mm_split(g, kLayerSplit) : 1, part, s);
  for (int i = 0; i < g.nseg; ++i) {
    const MmSeg& q = g.seg[i];
    const int end = i + 1 < g.nseg ? g.seg[i + 1].off : (g.seg_k ? g.K : g.N);
    const Gemm e = g.seg_k ? Gemm{g.M, g.N, end - q.off, q.A, q.sam, q.sak, q.B, q.sbk, q.sbn, (float*)g.C, g.ldc,
                                  g.accumulate || i > 0}
                           : Gemm{g.M, end - q.off, g.K, g.A, g.sam, g.sak, q.B, q.sbk, q.sbn, (float*)q.C, q.ldc,
                                  g.accumulate};
    const hipError_t r = gemm_exact(e, true, true, split ? part : nullptr, s);
    if (r != hipSuccess) return r;
  }
  return hipSuccess;
}

// The layer's GEMMs take 16-byte rows: with bf16 I/O the width C must be a
// multiple of 8 (the head widths always are).
bool layer_shapes_ok(const Dims& dm) { return dm.io != IO_BF16 || dm.C % 8 == 0; }

bool layer_weights_ok(const void* const* ps, int n) {
  for (int i = 0; i < n; ++i)
    if (!ps[i] || !aligned16(ps[i])) return false;
  return true;
}

}  // namespace

extern "C" {

int nsa_abi_version(void) { return NSA_ABI_VERSION; }

const char* nsa_status_str(nsa_status s) {
  switch (s) {
    case NSA_OK: return "ok";
    case NSA_ERR_INVALID_ARG: return "invalid argument";
    case NSA_ERR_UNSUPPORTED: return "unsupported configuration or device";
    case NSA_ERR_WORKSPACE: return "workspace missing or too small";
    case NSA_ERR_HIP: return "HIP runtime error";
    case NSA_ERR_INTERNAL: return "internal error";
    case NSA_ERR_SCRATCH: return "problem larger than the library's static scratch buffer";
  }
  return "unknown status";
}

nsa_status nsa_workspace_size(const nsa_params* p, nsa_op op, size_t* bytes) {
  try {
    if (!bytes) return NSA_ERR_INVALID_ARG;
    Dims dm;
    nsa_status st = make_dims(p, &dm);
    if (st != NSA_OK) return st;
    PrefillWs w;
    switch (op) {
      case NSA_OP_FWD_PREFILL: *bytes = plan_prefill(dm, nullptr, &w); return NSA_OK;
      case NSA_OP_FWD_DECODE: *bytes = decode_ws_bytes(dm); return NSA_OK;
      case NSA_OP_BWD: *bytes = bwd_ws_bytes(dm); return NSA_OK;
      case NSA_OP_COMPRESS: *bytes = phi_ws(dm) > 0 ? phi_ws(dm) : 256; return NSA_OK;
      case NSA_OP_DENSE: *bytes = dense_ws_bytes(dm); return NSA_OK;
      case NSA_OP_APPEND: *bytes = append_ws_bytes(dm) > 0 ? append_ws_bytes(dm) : 256; return NSA_OK;
      case NSA_OP_DENSE_BWD: *bytes = dense_bwd_ws_bytes(dm); return NSA_OK;
      case NSA_OP_LAYER_FWD: *bytes = plan_prefill(dm, nullptr, &w); return NSA_OK;
      case NSA_OP_LAYER_BWD: *bytes = plan_layer_bwd(dm, nullptr, nullptr); return NSA_OK;
    }
    return NSA_ERR_INVALID_ARG;
  } catch (...) {
    return NSA_ERR_INTERNAL;
  }
}

nsa_status nsa_compress(const nsa_params* p, int is_value, const void* x, const nsa_phi_weights* phi,
                        void* out, void* ws, size_t ws_bytes, void* stream) {
  try {
    Dims dm;
    nsa_status st = make_dims(p, &dm);
    if (st != NSA_OK) return st;
    if (!x || !out || !aligned16(x) || !aligned16(out)) return NSA_ERR_INVALID_ARG;
    if (dm.hidden && (!phi || !phi_ok(*phi))) return NSA_ERR_INVALID_ARG;
    const size_t need = phi_ws(dm);
    if (ws_bytes < need || (need && !ws) || !aligned16(ws)) return NSA_ERR_WORKSPACE;
    if ((st = check_device()) != NSA_OK) return st;
    const int D = is_value ? dm.dv : dm.dk;
    return hip_status(run_compress(dm, D, x, phi, out, nullptr, ws, (hipStream_t)stream));
  } catch (...) {
    return NSA_ERR_INTERNAL;
  }
}

// check_only: run every check (the device's included) and return without
// enqueuing anything.
static nsa_status prefill_impl(const nsa_params* p, const nsa_prefill_args* a, void* ws, size_t ws_bytes,
                               void* stream, void* const* events, int n_events, bool check_only = false) {
  try {
    Dims dm;
    nsa_status st = make_dims(p, &dm);
    if (st != NSA_OK) return st;
    if (!a) return NSA_ERR_INVALID_ARG;
    if (events && n_events < kPrefillStages + 1) return NSA_ERR_INVALID_ARG;
    const void* req[] = {a->q, a->k, a->v, a->x, a->w_gate, a->o};
    for (const void* r : req)
      if (!r || !aligned16(r)) return NSA_ERR_INVALID_ARG;
    const void* opt[] = {a->k_cmp, a->v_cmp, a->lse, a->idx, a->o_branch, a->p_slc, a->gates};
    for (const void* r : opt)
      if (r && !aligned16(r)) return NSA_ERR_INVALID_ARG;
    bool given_cmp = false;
    if (!all_or_none({a->k_cmp_in, a->v_cmp_in}, &given_cmp)) return NSA_ERR_INVALID_ARG;
    // phi runs when there is a complete block and no compressed keys are given
    const bool run_phi = dm.ncmp > 0 && !given_cmp;
    if (dm.hidden && run_phi && (!phi_ok(a->phi_k) || !phi_ok(a->phi_v))) return NSA_ERR_INVALID_ARG;
    if (!gate_ok(dm, a->gate_mlp)) return NSA_ERR_INVALID_ARG;
    bool split = false;
    if (!all_or_none({a->k_slc, a->v_slc, a->k_win, a->v_win}, &split)) return NSA_ERR_INVALID_ARG;
    PrefillWs w;
    const size_t need = plan_prefill(dm, nullptr, &w);
    if (ws_bytes < need || !ws || !aligned16(ws)) return NSA_ERR_WORKSPACE;
    if ((st = check_device()) != NSA_OK) return st;
    if (check_only) return NSA_OK;
    plan_prefill(dm, ws, &w);
    hipStream_t s = (hipStream_t)stream;
    Stages sg(events, s);
    const size_t BTH = (size_t)dm.B * dm.T * dm.Hq;
    const size_t es = esize(dm);
    float* gates = a->gates ? (float*)a->gates : (float*)w.gates;
    const void* kc = given_cmp ? a->k_cmp_in : (a->k_cmp ? a->k_cmp : w.kc);
    const void* vc = given_cmp ? a->v_cmp_in : (a->v_cmp ? a->v_cmp : w.vc);
    float* lse = a->lse ? (float*)a->lse : (float*)w.lse;
    int* idx = a->idx ? (int*)a->idx : (int*)w.idx;
    // branch outputs: fp32 when saved for the backward, else I/O type in the workspace
    const int o_f32 = a->o_branch ? 1 : 0;
    const size_t obs = o_f32 ? 4 : es;
    char* ob = a->o_branch ? (char*)a->o_branch : (char*)w.ob;
    void* o_cmp = ob;
    void* o_slc = ob + BTH * dm.dv * obs;
    void* o_win = a->o_branch ? ob + 2 * BTH * dm.dv * obs : nullptr;
    if (sg.mark() ||
        launch_gate_mlp(dm, dm.B * dm.T, a->x, a->w_gate, GateMlp{a->gate_mlp.w1, a->gate_mlp.b1, a->gate_mlp.b2},
                        (float*)w.gh, nullptr, gates, s) != hipSuccess)
      return NSA_ERR_HIP;
    if (run_phi) {
      if (sg.mark() || run_compress(dm, dm.dk, a->k, &a->phi_k, (void*)kc, nullptr, w.phi, s) != hipSuccess)
        return NSA_ERR_HIP;
      if (sg.mark() || run_compress(dm, dm.dv, a->v, &a->phi_v, (void*)vc, w.vct, w.phi, s) != hipSuccess)
        return NSA_ERR_HIP;
    } else {
      // the caller's compressed keys and values (or none: no block is
      // complete): V_cmp^T for the compressed pass, copies for the saved
      // outputs
      const size_t kb = (size_t)dm.B * dm.ncmp * dm.Hkv * dm.dk * es, vb = (size_t)dm.B * dm.ncmp * dm.Hkv * dm.dv * es;
      if (sg.mark() || (a->k_cmp && kb && hipMemcpyAsync(a->k_cmp, kc, kb, hipMemcpyDeviceToDevice, s) != hipSuccess))
        return NSA_ERR_HIP;
      if (sg.mark() || (a->v_cmp && vb && hipMemcpyAsync(a->v_cmp, vc, vb, hipMemcpyDeviceToDevice, s) != hipSuccess) ||
          (vb && launch_transpose_seq(dm, dm.B, dm.ncmp, dm.Hkv, dm.dv, dm.ncmp_pad, vc, w.vct, s) != hipSuccess))
        return NSA_ERR_HIP;
    }
    const void* ks = split ? a->k_slc : a->k;
    const void* vs = split ? a->v_slc : a->v;
    const void* kw = split ? a->k_win : a->k;
    const void* vw = split ? a->v_win : a->v;
    if (sg.mark() || launch_transpose_seq(dm, dm.B, dm.T, dm.Hkv, dm.dv, dm.Tp, vw, w.vt, s) != hipSuccess ||
        launch_kv_frag(dm, ks, vs, w.kvf, s) != hipSuccess)
      return NSA_ERR_HIP;
    CmpArgs ca;
    ca.q = a->q; ca.kc = kc; ca.vct = w.vct; ca.lse = lse; ca.o = o_cmp; ca.p_slc = (float*)a->p_slc; ca.idx = idx;
    ca.o_f32 = o_f32;
    if (sg.mark() || launch_cmp_lse(dm, ca, s) != hipSuccess) return NSA_ERR_HIP;
    if (sg.mark() || launch_cmp_out_topn(dm, ca, s) != hipSuccess) return NSA_ERR_HIP;
    SlcArgs sa;
    sa.q = a->q; sa.kvf = w.kvf; sa.idx = idx; sa.o = o_slc; sa.lse = lse + BTH; sa.o_f32 = o_f32;
    if (sg.mark() || launch_slc(dm, sa, s) != hipSuccess) return NSA_ERR_HIP;
    WinArgs wa{};
    wa.q = a->q; wa.k = kw; wa.vt = w.vt; wa.o_cmp = o_cmp; wa.o_slc = o_slc; wa.gates = gates;
    wa.o_win = o_win; wa.lse = lse + 2 * BTH; wa.o = a->o; wa.o_f32 = o_f32;
    if (sg.mark() || launch_win_combine(dm, wa, s) != hipSuccess) return NSA_ERR_HIP;
    if (sg.mark()) return NSA_ERR_HIP;
    // measurement only: the selected branch's gather without its arithmetic,
    // timed by one more event; its one word per wave goes to the V^T copy,
    // which no stage reads any more
    if (events && n_events >= kPrefillStages + 2) {
      if (slc_gather_sink_bytes(dm) > (size_t)dm.B * dm.Hkv * dm.dv * dm.Tp * es) return NSA_ERR_INTERNAL;
      if (launch_slc_gather(dm, sa, w.vt, s) != hipSuccess || sg.mark()) return NSA_ERR_HIP;
    }
    return NSA_OK;
  } catch (...) {
    return NSA_ERR_INTERNAL;
  }
}

nsa_status nsa_fwd_prefill(const nsa_params* p, const nsa_prefill_args* a, void* ws, size_t ws_bytes,
                           void* stream) {
  return prefill_impl(p, a, ws, ws_bytes, stream, nullptr, 0);
}

nsa_status nsa_fwd_prefill_timed(const nsa_params* p, const nsa_prefill_args* a, void* ws, size_t ws_bytes,
                                 void* stream, void* const* events, int n_events) {
  if (!events) return NSA_ERR_INVALID_ARG;
  return prefill_impl(p, a, ws, ws_bytes, stream, events, n_events);
}

// Dense causal attention: the window kernel with a window covering every key
// and no gated combine.
nsa_status nsa_dense_fwd(const nsa_params* p, const nsa_dense_args* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    Dims dm;
    nsa_status st = make_dims(p, &dm);
    if (st != NSA_OK) return st;
    if (!a) return NSA_ERR_INVALID_ARG;
    const void* req[] = {a->q, a->k, a->v, a->o};
    for (const void* r : req)
      if (!r || !aligned16(r)) return NSA_ERR_INVALID_ARG;
    if (a->lse && !aligned16(a->lse)) return NSA_ERR_INVALID_ARG;
    if (ws_bytes < dense_ws_bytes(dm) || !ws || !aligned16(ws)) return NSA_ERR_WORKSPACE;
    if ((st = check_device()) != NSA_OK) return st;
    dm.w = dm.T;
    hipStream_t s = (hipStream_t)stream;
    if (launch_transpose_seq(dm, dm.B, dm.T, dm.Hkv, dm.dv, dm.Tp, a->v, ws, s) != hipSuccess) return NSA_ERR_HIP;
    WinArgs wa{};
    wa.q = a->q; wa.k = a->k; wa.vt = ws; wa.o = a->o; wa.lse = (float*)a->lse; wa.dense = 1;
    if (launch_win_combine(dm, wa, s) != hipSuccess) return NSA_ERR_HIP;
    return NSA_OK;
  } catch (...) {
    return NSA_ERR_INTERNAL;
  }
}

nsa_status nsa_decode_append(const nsa_params* p, const nsa_append_args* a, void* ws, size_t ws_bytes,
                             void* stream) {
  try {
    Dims dm;
    nsa_status st = make_dims(p, &dm);
    if (st != NSA_OK) return st;
    if (!a) return NSA_ERR_INVALID_ARG;
    const void* req[] = {a->k_new, a->v_new, a->seq_lens, a->k_cache, a->v_cache};
    for (const void* r : req)
      if (!r || !aligned16(r)) return NSA_ERR_INVALID_ARG;
    if (dm.ncmp > 0 && (!a->k_cmp_cache || !a->v_cmp_cache || !aligned16(a->k_cmp_cache) ||
                        !aligned16(a->v_cmp_cache) || a->cmp_cache_cap < dm.ncmp))
      return NSA_ERR_INVALID_ARG;
    if (dm.hidden && (!phi_ok(a->phi_k) || !phi_ok(a->phi_v))) return NSA_ERR_INVALID_ARG;
    bool slc = false, win = false;
    if (!all_or_none({a->k_slc_new, a->v_slc_new, a->k_slc_cache, a->v_slc_cache}, &slc) ||
        !all_or_none({a->k_win_new, a->v_win_new, a->k_win_cache, a->v_win_cache}, &win))
      return NSA_ERR_INVALID_ARG;
    const size_t need = append_ws_bytes(dm);
    if (ws_bytes < need || (need && !ws) || !aligned16(ws)) return NSA_ERR_WORKSPACE;
    if ((st = check_device()) != NSA_OK) return st;
    AppendArgs aa;
    aa.lens = a->seq_lens; aa.kn = a->k_new; aa.vn = a->v_new; aa.kc = a->k_cache; aa.vc = a->v_cache;
    aa.kn_slc = a->k_slc_new; aa.vn_slc = a->v_slc_new; aa.kc_slc = a->k_slc_cache; aa.vc_slc = a->v_slc_cache;
    aa.kn_win = a->k_win_new; aa.vn_win = a->v_win_new; aa.kc_win = a->k_win_cache; aa.vc_win = a->v_win_cache;
    aa.kcmp = a->k_cmp_cache; aa.vcmp = a->v_cmp_cache; aa.cap = a->cmp_cache_cap;
    aa.phi_k = {a->phi_k.pe, a->phi_k.w1, a->phi_k.b1, a->phi_k.w2, a->phi_k.b2};
    aa.phi_v = {a->phi_v.pe, a->phi_v.w1, a->phi_v.b1, a->phi_v.w2, a->phi_v.b2};
    aa.h = (float*)ws;
    return hip_status(launch_append(dm, aa, (hipStream_t)stream));
  } catch (...) {
    return NSA_ERR_INTERNAL;
  }
}

nsa_status nsa_dense_bwd(const nsa_params* p, const nsa_dense_bwd_args* a, void* ws, size_t ws_bytes,
                         void* stream) {
  try {
    Dims dm;
    nsa_status st = make_dims(p, &dm);
    if (st != NSA_OK) return st;
    if (!a) return NSA_ERR_INVALID_ARG;
    const void* req[] = {a->q, a->k, a->v, a->o, a->lse, a->d_o, a->dq, a->dk, a->dv};
    for (const void* r : req)
      if (!r || !aligned16(r)) return NSA_ERR_INVALID_ARG;
    if (!dense_bwd_supported(dm)) return NSA_ERR_UNSUPPORTED;
    if (ws_bytes < dense_bwd_ws_bytes(dm) || !ws || !aligned16(ws)) return NSA_ERR_WORKSPACE;
    if ((st = check_device()) != NSA_OK) return st;
    return hip_status(launch_dense_bwd(dm, a, ws, (hipStream_t)stream));
  } catch (...) {
    return NSA_ERR_INTERNAL;
  }
}

int nsa_prefill_stage_count(void) { return kPrefillStages; }
int nsa_decode_stage_count(void) { return kDecodeStages; }
int nsa_bwd_stage_count(void) { return bwd_stage_count(); }

// static_scratch: run in the library's per-GPU static buffer instead of the
// caller's workspace (ws, ws_bytes unused).
static nsa_status decode_impl(const nsa_params* p, const nsa_decode_args* a, void* ws, size_t ws_bytes,
                              void* stream, void* const* events, int n_events, bool static_scratch = false) {
  try {
    Dims dm;
    nsa_status st = make_dims(p, &dm);
    if (st != NSA_OK) return st;
    if (!decode_fits(dm)) return NSA_ERR_UNSUPPORTED;
    if (!a) return NSA_ERR_INVALID_ARG;
    if (events && n_events < kDecodeStages + 1) return NSA_ERR_INVALID_ARG;
    const void* req[] = {a->q, a->k_cache, a->v_cache, a->x, a->w_gate, a->o};
    for (const void* r : req)
      if (!r || !aligned16(r)) return NSA_ERR_INVALID_ARG;
    if (dm.ncmp > 0 && (!a->k_cmp_cache || !a->v_cmp_cache || !aligned16(a->k_cmp_cache) ||
                        !aligned16(a->v_cmp_cache) || a->cmp_cache_cap < dm.ncmp))
      return NSA_ERR_INVALID_ARG;
    const void* opt[] = {a->idx, a->p_slc, a->lse, a->o_branch, a->seq_lens};
    for (const void* r : opt)
      if (r && !aligned16(r)) return NSA_ERR_INVALID_ARG;
    bool split = false;
    if (!all_or_none({a->k_win_cache, a->v_win_cache}, &split)) return NSA_ERR_INVALID_ARG;
    if (!gate_ok(dm, a->gate_mlp)) return NSA_ERR_INVALID_ARG;
    const size_t need = decode_ws_bytes(dm);
    if (static_scratch) {
      if (need > NSA_DECODE_STATIC_SCRATCH_BYTES) return NSA_ERR_SCRATCH;
    } else if (ws_bytes < need || !ws || !aligned16(ws)) {
      return NSA_ERR_WORKSPACE;
    }
    if ((st = check_device()) != NSA_OK) return st;
    if (static_scratch && decode_static_scratch(&ws) != hipSuccess) return NSA_ERR_HIP;
    return hip_status(launch_decode(dm, a, ws, (hipStream_t)stream, events));
  } catch (...) {
    return NSA_ERR_INTERNAL;
  }
}

nsa_status nsa_fwd_decode(const nsa_params* p, const nsa_decode_args* a, void* ws, size_t ws_bytes,
                          void* stream) {
  return decode_impl(p, a, ws, ws_bytes, stream, nullptr, 0);
}

nsa_status nsa_fwd_decode_noalloc(const nsa_params* p, const nsa_decode_args* a, void* stream) {
  return decode_impl(p, a, nullptr, 0, stream, nullptr, 0, true);
}

nsa_status nsa_fwd_decode_timed(const nsa_params* p, const nsa_decode_args* a, void* ws, size_t ws_bytes,
                                void* stream, void* const* events, int n_events) {
  if (!events) return NSA_ERR_INVALID_ARG;
  return decode_impl(p, a, ws, ws_bytes, stream, events, n_events);
}

static nsa_status bwd_impl(const nsa_params* p, const nsa_bwd_args* a, void* ws, size_t ws_bytes, void* stream,
                           void* const* events, int n_events, bool check_only = false) {
  try {
    Dims dm;
    nsa_status st = make_dims(p, &dm);
    if (st != NSA_OK) return st;
    if (!a) return NSA_ERR_INVALID_ARG;
    if (events && n_events < bwd_stage_count() + 1) return NSA_ERR_INVALID_ARG;
    const void* req[] = {a->q, a->k, a->v, a->x, a->w_gate, a->lse, a->idx, a->d_o,
                         a->dq, a->dk, a->dv, a->dw_gate};
    for (const void* r : req)
      if (!r || !aligned16(r)) return NSA_ERR_INVALID_ARG;
    if (dm.ncmp > 0 && (!a->k_cmp || !a->v_cmp || !aligned16(a->k_cmp) || !aligned16(a->v_cmp)))
      return NSA_ERR_INVALID_ARG;
    if (dm.hidden) {
      if (!phi_ok(a->phi_k) || !phi_ok(a->phi_v)) return NSA_ERR_INVALID_ARG;
      const void* g[] = {a->d_phi_k.pe, a->d_phi_k.w1, a->d_phi_k.b1, a->d_phi_k.w2, a->d_phi_k.b2,
                         a->d_phi_v.pe, a->d_phi_v.w1, a->d_phi_v.b1, a->d_phi_v.w2, a->d_phi_v.b2};
      for (const void* r : g)
        if (!r || !aligned16(r)) return NSA_ERR_INVALID_ARG;
    }
    if (!gate_ok(dm, a->gate_mlp)) return NSA_ERR_INVALID_ARG;
    if (dm.Cg && (!a->d_gate_mlp.w1 || !a->d_gate_mlp.b1 || !a->d_gate_mlp.b2 || !aligned16(a->d_gate_mlp.w1) ||
                  !aligned16(a->d_gate_mlp.b1) || !aligned16(a->d_gate_mlp.b2)))
      return NSA_ERR_INVALID_ARG;
    if (a->dx && !aligned16(a->dx)) return NSA_ERR_INVALID_ARG;
    bool split = false, split_out = false;
    if (!all_or_none({a->k_slc, a->v_slc, a->k_win, a->v_win}, &split) ||
        !all_or_none({a->dk_slc, a->dv_slc, a->dk_win, a->dv_win}, &split_out) || split != split_out)
      return NSA_ERR_INVALID_ARG;
    const size_t need = bwd_ws_bytes(dm);
    if (ws_bytes < need || !ws || !aligned16(ws)) return NSA_ERR_WORKSPACE;
    if ((st = check_device()) != NSA_OK) return st;
    if (check_only) return NSA_OK;
    return hip_status(launch_bwd(dm, a, ws, (hipStream_t)stream, events));
  } catch (...) {
    return NSA_ERR_INTERNAL;
  }
}

nsa_status nsa_bwd(const nsa_params* p, const nsa_bwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  return bwd_impl(p, a, ws, ws_bytes, stream, nullptr, 0);
}

nsa_status nsa_bwd_timed(const nsa_params* p, const nsa_bwd_args* a, void* ws, size_t ws_bytes, void* stream,
                         void* const* events, int n_events) {
  if (!events) return NSA_ERR_INVALID_ARG;
  return bwd_impl(p, a, ws, ws_bytes, stream, events, n_events);
}

nsa_status nsa_layer_fwd(const nsa_params* p, const nsa_layer_args* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    Dims dm;
    nsa_status st = make_dims(p, &dm);
    if (st != NSA_OK) return st;
    if (!a) return NSA_ERR_INVALID_ARG;
    const void* req[] = {a->h, a->w_q, a->w_k, a->w_v, a->w_o, a->y, a->q, a->k, a->v, a->o};
    if (!layer_weights_ok(req, 10)) return NSA_ERR_INVALID_ARG;
    nsa_prefill_args pa{};
    pa.q = a->q; pa.k = a->k; pa.v = a->v; pa.x = a->h; pa.w_gate = a->w_gate;
    pa.phi_k = a->phi_k; pa.phi_v = a->phi_v; pa.o = a->o;
    pa.k_cmp = a->k_cmp; pa.v_cmp = a->v_cmp; pa.lse = a->lse; pa.idx = a->idx; pa.o_branch = a->o_branch;
    pa.gate_mlp = a->gate_mlp;
    if ((st = prefill_impl(p, &pa, ws, ws_bytes, stream, nullptr, 0, true)) != NSA_OK) return st;
    if (!layer_shapes_ok(dm)) return NSA_ERR_UNSUPPORTED;
    const int ntok = dm.B * dm.T, C = dm.C, bo = dm.io == IO_BF16;
    const int nq = dm.Hq * dm.dk, nk = dm.Hkv * dm.dk, nv = dm.Hkv * dm.dv, no = dm.Hq * dm.dv;
    hipStream_t s = (hipStream_t)stream;
    // [q | k | v] = h [w_q | w_k | w_v] in one launch (outputs in the I/O type)
    MmArgs gx{ntok, nq + nk + nv, C, a->h, C, 1, nullptr, nq, 1, nullptr, 0, 0, bo};
    gx.nseg = 3;
    gx.seg[0] = MmSeg{nullptr, 0, 0, a->w_q, nq, 1, a->q, nq, 0};
    gx.seg[1] = MmSeg{nullptr, 0, 0, a->w_k, nk, 1, a->k, nk, nq};
    gx.seg[2] = MmSeg{nullptr, 0, 0, a->w_v, nv, 1, a->v, nv, nq + nk};
    if (layer_gemm_seg(dm, gx, false, false, false, nullptr, s) != hipSuccess) return NSA_ERR_HIP;
    if ((st = prefill_impl(p, &pa, ws, ws_bytes, stream, nullptr, 0)) != NSA_OK) return st;
    // y = o w_o
    const MmArgs gy{ntok, C, no, a->o, no, 1, a->w_o, C, 1, a->y, C, 0, bo};
    return hip_status(layer_gemm(dm, gy, false, false, false, nullptr, s));
  } catch (...) {
    return NSA_ERR_INTERNAL;
  }
}

nsa_status nsa_layer_bwd(const nsa_params* p, const nsa_layer_bwd_args* a, void* ws, size_t ws_bytes,
                         void* stream) {
  try {
    Dims dm;
    nsa_status st = make_dims(p, &dm);
    if (st != NSA_OK) return st;
    if (!a) return NSA_ERR_INVALID_ARG;
    const void* req[] = {a->h, a->w_q, a->w_k, a->w_v, a->w_o, a->q, a->k, a->v, a->o, a->dy,
                         a->dh, a->dw_q, a->dw_k, a->dw_v, a->dw_o};
    if (!layer_weights_ok(req, 15)) return NSA_ERR_INVALID_ARG;
    const size_t need = plan_layer_bwd(dm, nullptr, nullptr);
    if (ws_bytes < need || !ws || !aligned16(ws)) return NSA_ERR_WORKSPACE;
    LayerBwdWs w;
    plan_layer_bwd(dm, ws, &w);
    nsa_bwd_args ba{};
    ba.q = a->q; ba.k = a->k; ba.v = a->v; ba.x = a->h; ba.w_gate = a->w_gate;
    ba.phi_k = a->phi_k; ba.phi_v = a->phi_v;
    ba.k_cmp = a->k_cmp; ba.v_cmp = a->v_cmp; ba.lse = a->lse; ba.idx = a->idx; ba.o_branch = a->o_branch;
    ba.d_o = w.d_o; ba.dq = w.dq; ba.dk = w.dk; ba.dv = w.dv; ba.dw_gate = a->dw_gate;
    ba.d_phi_k = a->d_phi_k; ba.d_phi_v = a->d_phi_v;
    ba.gate_mlp = a->gate_mlp; ba.d_gate_mlp = a->d_gate_mlp; ba.dx = a->dh;
    const size_t op_bytes = bwd_ws_bytes(dm);
    if ((st = bwd_impl(p, &ba, w.op_ws, op_bytes, stream, nullptr, 0, true)) != NSA_OK) return st;
    if (!layer_shapes_ok(dm)) return NSA_ERR_UNSUPPORTED;
    const int ntok = dm.B * dm.T, C = dm.C, bo = dm.io == IO_BF16;
    const int nq = dm.Hq * dm.dk, nk = dm.Hkv * dm.dk, nv = dm.Hkv * dm.dv, no = dm.Hq * dm.dv;
    hipStream_t s = (hipStream_t)stream;
    // dO = dy w_o^T (I/O type), dW_o = o^T dy (fp32)
    const MmArgs gdo{ntok, no, C, a->dy, C, 1, a->w_o, 1, C, w.d_o, no, 0, bo};
    const MmArgs gwo{no, C, ntok, a->o, 1, no, a->dy, C, 1, a->dw_o, C, 0, 0};
    if (layer_gemm(dm, gdo, false, false, false, nullptr, s) != hipSuccess ||
        layer_gemm(dm, gwo, false, false, true, w.part, s) != hipSuccess)
      return NSA_ERR_HIP;
    // the operator's backward; its dx (the gate path) initialises dh
    if ((st = bwd_impl(p, &ba, w.op_ws, op_bytes, stream, nullptr, 0)) != NSA_OK) return st;
    // [dW_q | dW_k | dW_v] = h^T [dq | dk | dv] (fp32) in one launch, split
    // over the tokens
    MmArgs gw{C, nq + nk + nv, ntok, a->h, 1, C, nullptr, nq, 1, nullptr, 0, 0, 0};
    gw.nseg = 3;
    gw.seg[0] = MmSeg{nullptr, 0, 0, w.dq, nq, 1, a->dw_q, nq, 0};
    gw.seg[1] = MmSeg{nullptr, 0, 0, w.dk, nk, 1, a->dw_k, nk, nq};
    gw.seg[2] = MmSeg{nullptr, 0, 0, w.dv, nv, 1, a->dw_v, nv, nq + nk};
    // dh += [dq | dk | dv] [w_q | w_k | w_v]^T in one launch, the contraction
    // running over the three segments (dq, dk, dv are fp32)
    MmArgs gh{ntok, C, nq + nk + nv, nullptr, nq, 1, nullptr, 1, nq, a->dh, C, 1, 0};
    gh.nseg = 3;
    gh.seg_k = 1;
    gh.seg[0] = MmSeg{w.dq, nq, 1, a->w_q, 1, nq, nullptr, 0, 0};
    gh.seg[1] = MmSeg{w.dk, nk, 1, a->w_k, 1, nk, nullptr, 0, nq};
    gh.seg[2] = MmSeg{w.dv, nv, 1, a->w_v, 1, nv, nullptr, 0, nq + nk};
    if (layer_gemm_seg(dm, gw, false, true, true, w.part, s) != hipSuccess ||
        layer_gemm_seg(dm, gh, true, false, false, nullptr, s) != hipSuccess)
      return NSA_ERR_HIP;
    return NSA_OK;
  } catch (...) {
    return NSA_ERR_INTERNAL;
  }
}

}  // extern "C"
