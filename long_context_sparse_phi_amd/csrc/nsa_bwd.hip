// Backward pass of NSA on gfx950 with the selected blocks held fixed.
//
// For every branch c (cmp, slc, win) with dO_c = g_c dO and the forward's
// log-sum-exp saved per row:
//   P = exp(scale q k^T - lse_c);  dP = dO_c v^T;  D_c = rowsum(dO_c * O_c);
//   dS = P * (dP - D_c);  dq += scale dS k;  dk += scale dS^T q;  dv += P^T dO_c.
// Gate: dg_c = <dO, O_c> = sum_k P_k (dO . v_k), evaluated from the recomputed
// probabilities so that no rounded copy of O_c enters it; dz = dg g (1 - g),
// dW_g = x^T dz.  The compressed
// keys/values receive dK_cmp / dV_cmp, which flow back through phi to k, v
// and phi's parameters.  No gradient flows through the scores or the
// top-n selection (the natively trainable formulation of the NSA pages, with
// the selection treated as a discrete choice).
//
// Work decomposition (deterministic, no floating-point atomics):
//   * k_bwd_dq: one wave per (position, KV group) holding the G heads as the
//     16 MFMA columns; it walks the compressed keys, the selected blocks and
//     the window keys and accumulates dq^T = K^T dS^T in registers.
//   * k_bwd_kv: one wave per 16 keys; it walks the query positions that see
//     those keys (a range for cmp and win, the reverse index of a selected
//     block for slc), two positions x 16 heads per step, and accumulates
//     dK^T = Q^T dS and dV^T = dO_c^T P.  Long query ranges are split into
//     segments whose partial sums are added in a fixed order afterwards.
//   * The reverse index (positions that selected each block, ascending) is
//     built by a per-chunk histogram, a scan and an ordered fill.
//   * phi and the gate projection go through a strided fp32 MFMA GEMM.
#include "../../include/nsa.h"
#include "nsa_common.hpp"
#include "nsa_kernels.hpp"

namespace nsa {

int bwd_stage_count() { return 8; }

constexpr int kSegCmp = 1024;    // query positions per compressed-key segment
constexpr int kSegSlc = 1024;    // list entries per selected-block segment
constexpr int kRevChunk = 256;   // positions per reverse-index chunk

struct BwdPlan {
  int nkt_cmp;     // 16-key tiles of the compressed keys
  int nseg_cmp;    // segments per compressed key tile (upper bound)
  int nchunk;      // reverse-index chunks
  int nseg_slc;    // segments per selected block (upper bound)
  int max_slc_seg; // segment slots per (b, g)
  int Ts;          // stride of the padded transposed q / dO: T*16
};

static BwdPlan bwd_plan(const Dims& dm) {
  BwdPlan p;
  p.nkt_cmp = (dm.ncmp + 15) / 16;
  p.nseg_cmp = (dm.T + kSegCmp - 1) / kSegCmp;
  p.nchunk = (dm.T + kRevChunk - 1) / kRevChunk;
  p.nseg_slc = (dm.T + kSegSlc - 1) / kSegSlc;
  p.max_slc_seg = dm.nsel + (int)(((long long)dm.T * dm.n + kSegSlc - 1) / kSegSlc);
  p.Ts = dm.T * 16;
  return p;
}

struct BwdBufs {
  float* gates;    // [B,T,Hq,3]
  float* Dc;       // [3,B,T,Hq]
  float* dz;       // [B,T,Hq,3]
  void* kt;        // [B,Hkv,dk,Tp]
  void* kct;       // [B,Hkv,dk,ncmp_pad]
  void* qt;        // [B,Hkv,dk,T*16]
  void* dot;       // [B,Hkv,dv,T*16]
  float* dkc;      // [B,Hkv,ncmp,dk]
  float* dvc;      // [B,Hkv,ncmp,dv]
  float* part_cmp; // [B*Hkv*nkt*nseg][16][dk+dv]
  int* hist;       // [B*Hkv][nchunk][nsel]
  int* offc;       // [B*Hkv][nchunk][nsel]
  int* cnt;        // [B*Hkv][nsel]
  int* lstart;     // [B*Hkv][nsel]
  int* segoff;     // [B*Hkv][nsel]
  int* list;       // [B*Hkv][T*n]
  float* part_slc; // [B*Hkv*max_slc_seg][ls][dk+dv]
  // phi
  void* w1t;       // [H, l*D]   io
  void* w2t;       // [D, H]     io
  float* y;        // GEMM1 output
  float* act;      // [R,H] pre-activation
  float* hid;      // [R,H] gelu(act)
  float* dh;       // [R,H]
  float* du;       // [R,l*D]
};

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t bwd_carve(const Dims& dm, void* ws, BwdBufs* w) {
  const BwdPlan p = bwd_plan(dm);
  char* base = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t bytes) { void* r = base ? base + off : nullptr; off += al256(bytes); return r; };
  const size_t es = dm.io == IO_BF16 ? 2 : 4;
  const size_t BTH = (size_t)dm.B * dm.T * dm.Hq, BG = (size_t)dm.B * dm.Hkv;
  w->gates = (float*)take(BTH * 3 * 4);
  w->Dc = (float*)take(3 * BTH * 4);
  w->dz = (float*)take(BTH * 3 * 4);
  w->kt = take(BG * dm.dk * dm.Tp * es);
  w->kct = take(BG * dm.dk * dm.ncmp_pad * es);
  w->qt = take(BG * dm.dk * p.Ts * es);
  w->dot = take(BG * dm.dv * p.Ts * es);
  w->dkc = (float*)take(BG * dm.ncmp * dm.dk * 4);
  w->dvc = (float*)take(BG * dm.ncmp * dm.dv * 4);
  w->part_cmp = (float*)take(BG * p.nkt_cmp * p.nseg_cmp * 16 * (dm.dk + dm.dv) * 4);
  w->hist = (int*)take(BG * p.nchunk * dm.nsel * 4);
  w->offc = (int*)take(BG * p.nchunk * dm.nsel * 4);
  w->cnt = (int*)take(BG * dm.nsel * 4);
  w->lstart = (int*)take(BG * dm.nsel * 4);
  w->segoff = (int*)take(BG * dm.nsel * 4);
  w->list = (int*)take(BG * dm.T * dm.n * 4);
  w->part_slc = (float*)take(BG * p.max_slc_seg * dm.ls * (dm.dk + dm.dv) * 4);
  if (dm.hidden) {
    const int D = dm.dk > dm.dv ? dm.dk : dm.dv;
    const int R = dm.l / dm.d;
    const size_t rows = BG * dm.ncmp;
    const size_t nsub = dm.ncmp > 0 ? dm.ncmp + R - 1 : 0;
    w->w1t = take((size_t)dm.hidden * dm.l * D * es);
    w->w2t = take((size_t)D * dm.hidden * es);
    w->y = (float*)take((BG * nsub + R) * R * dm.hidden * 4);
    w->act = (float*)take(rows * dm.hidden * 4);
    w->hid = (float*)take(rows * dm.hidden * 4);
    w->dh = (float*)take(rows * dm.hidden * 4);
    w->du = (float*)take(rows * dm.l * D * 4);
  }
  return off;
}

size_t bwd_ws_bytes(const Dims& dm) {
  BwdBufs w;
  return bwd_carve(dm, nullptr, &w);
}

struct BwdArgs {
  const void *q, *k, *v, *x, *wg, *kc, *vc, *d_o;
  const float* lse;  // [3,B,T,Hq] natural log
  const int* idx;    // [B,T,Hkv,n]
  float *dq, *dk, *dv, *dwg;
  BwdBufs w;
  BwdPlan pl;
};

// q / dO [B,T,Hq,D] -> [B,Hkv,D,T,16] with heads >= G zero-filled.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose_heads(Dims dm, int D, const T* __restrict__ src,
                                                         T* __restrict__ dst) {
  __shared__ float tile[64][65];
  const int bg = blockIdx.z, b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int r0 = blockIdx.x * 64;   // flattened (t, h16) index
  const int f0 = blockIdx.y * 64;
  const int Ts = dm.T * 16;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i >> 6, ff = i & 63, rf = r0 + rr, f = f0 + ff;
    const int t = rf >> 4, h = rf & 15;
    float v = 0.f;
    if (rf < Ts && f < D && h < dm.G) v = to_f32(src[((size_t)(b * dm.T + t) * dm.Hq + g * dm.G + h) * D + f]);
    tile[rr][ff] = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int ff = i >> 6, rr = i & 63, rf = r0 + rr, f = f0 + ff;
    if (f < D && rf < Ts) dst[((size_t)bg * D + f) * Ts + rf] = from_f32<T>(tile[rr][ff]);
  }
}

// ---------------------------------------------------------------------------
// dq: one wave per (b, t, g); columns = the G heads.
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV>
struct DqState {
  Frag8<T> qf[DK / 32];
  Frag8<T> dof[DV / 32];
  f32x4 dq[DK / 16];
  float rs;   // row-sum pass: this lane's part of sum_k P_k (dO . v_k)
};

// One 32-key tile of one branch.  kbase/vbase: row pointers of key/value
// rows (row stride kstr/vstr, already offset by qd*8); ktb: transposed keys
// (row stride ld, already offset by qd*8).  Keys kt .. kt+31, valid when
// lo <= key < hi.  ROWSUM: accumulate sum_k P_k dP_k (dP = dO v^T, no gate),
// which equals <dO, O_c> exactly; otherwise accumulate dq^T += K^T dS^T.
template <typename T, int DK, int DV, bool ROWSUM>
__device__ __forceinline__ void dq_tile(DqState<T, DK, DV>& st, const T* kbase, size_t kstr, const T* vbase,
                                        size_t vstr, const T* ktb, size_t ld, int kt, int lo, int hi, int klim,
                                        int krow, int c16, int qd, float sc2, float lse2, float gc, float Dc) {
  f32x4 s[2], dp[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    s[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
    dp[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int key = min(kt + krow + sub * 4, klim - 1);
    const T* kp = kbase + (size_t)key * kstr;
    const T* vp = vbase + (size_t)key * vstr;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) mma(s[sub], load_frag(kp + ks * 32), st.qf[ks]);
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks) mma(dp[sub], load_frag(vp + ks * 32), st.dof[ks]);
  }
  float ds[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int key = kt + qd * 8 + e;
    const bool v = key >= lo && key < hi;
    const float p = v ? fast_exp2(s[e >> 2][e & 3] * sc2 - lse2) : 0.f;
    if (ROWSUM) st.rs += p * dp[e >> 2][e & 3];
    else ds[e] = p * (gc * dp[e >> 2][e & 3] - Dc);
  }
  if (!ROWSUM) {
    Frag8<T> dsf = to_frag<T>(ds);
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) mma(st.dq[dt], load_frag(ktb + (size_t)(dt * 16 + c16) * ld + kt), dsf);
  }
}

// ROWSUM = true: per row and branch, dg_c = sum_k P_k (dO . v_k) = <dO, O_c>,
// written as D_c = g_c dg_c and dz_c = dg_c g_c (1 - g_c).  ROWSUM = false: dq.
template <typename T, int DK, int DV, bool ROWSUM>
__global__ __launch_bounds__(256) void k_bwd_dq(Dims dm, BwdArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  const int ntiles = (dm.T + 3) / 4;
  int unit, tile;
  xcd_map(blockIdx.x, dm.B * dm.Hkv, ntiles, unit, tile);
  const int b = unit / dm.Hkv, g = unit % dm.Hkv;
  const int t = tile * 4 + wave;
  if (t >= dm.T) return;
  const int G = dm.G;
  const bool cv = c16 < G;
  const int hq = g * G + (cv ? c16 : 0);
  const size_t BTH = (size_t)dm.B * dm.T * dm.Hq;
  const size_t row = (size_t)(b * dm.T + t) * dm.Hq + hq;
  DqState<T, DK, DV> st;
  {
    const T* qp = (const T*)a.q + row * DK + qd * 8;
    const T* dp = (const T*)a.d_o + row * DV + qd * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) st.qf[ks] = cv ? load_frag(qp + ks * 32) : zero_frag<T>();
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks) st.dof[ks] = cv ? load_frag(dp + ks * 32) : zero_frag<T>();
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) st.dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.rs = 0.f;
  }
  const float sc2 = dm.scale * kLog2e;
  const int krow = (c16 >> 2) * 8 + (c16 & 3);
  float lse2[3], gc[3], Dc[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const float l = cv ? a.lse[c * BTH + row] : 0.f;
    lse2[c] = l == kNegInf ? 0.f : l * kLog2e;
    gc[c] = cv ? a.w.gates[row * 3 + c] : 0.f;
    Dc[c] = (cv && !ROWSUM) ? a.w.Dc[c * BTH + row] : 0.f;
  }
  float rsum[3] = {0.f, 0.f, 0.f};
  // compressed branch
  {
    const int nv = ncmp_visible(t, dm.l, dm.d);
    const T* kb = (const T*)a.kc + ((size_t)b * dm.ncmp * dm.Hkv + g) * DK + qd * 8;
    const T* vb = (const T*)a.vc + ((size_t)b * dm.ncmp * dm.Hkv + g) * DV + qd * 8;
    const T* ktb = (const T*)a.w.kct + (size_t)(b * dm.Hkv + g) * DK * dm.ncmp_pad + qd * 8;
    for (int kt = 0; kt < nv; kt += 32)
      dq_tile<T, DK, DV, ROWSUM>(st, kb, (size_t)dm.Hkv * DK, vb, (size_t)dm.Hkv * DV, ktb, dm.ncmp_pad, kt, 0,
                                 nv, dm.ncmp, krow, c16, qd, sc2, lse2[0], gc[0], Dc[0]);
    rsum[0] = st.rs;
    st.rs = 0.f;
  }
  const T* kb = (const T*)a.k + ((size_t)b * dm.T * dm.Hkv + g) * DK + qd * 8;
  const T* vb = (const T*)a.v + ((size_t)b * dm.T * dm.Hkv + g) * DV + qd * 8;
  const T* ktb = (const T*)a.w.kt + (size_t)(b * dm.Hkv + g) * DK * dm.Tp + qd * 8;
  // selected branch
  {
    const int* ids = a.idx + ((size_t)(b * dm.T + t) * dm.Hkv + g) * dm.n;
    for (int si = 0; si < dm.n; ++si) {
      const int j = ids[si];
      if (j < 0) break;
      const int kend = min((j + 1) * dm.ls, t + 1);
      for (int kt = j * dm.ls; kt < kend; kt += 32)
        dq_tile<T, DK, DV, ROWSUM>(st, kb, (size_t)dm.Hkv * DK, vb, (size_t)dm.Hkv * DV, ktb, dm.Tp, kt,
                                   j * dm.ls, kend, dm.T, krow, c16, qd, sc2, lse2[1], gc[1], Dc[1]);
    }
    rsum[1] = st.rs;
    st.rs = 0.f;
  }
  // window branch
  {
    const int lo = max(0, t - dm.w + 1);
    for (int kt = lo & ~31; kt <= t; kt += 32)
      dq_tile<T, DK, DV, ROWSUM>(st, kb, (size_t)dm.Hkv * DK, vb, (size_t)dm.Hkv * DV, ktb, dm.Tp, kt, lo, t + 1,
                                 dm.T, krow, c16, qd, sc2, lse2[2], gc[2], Dc[2]);
    rsum[2] = st.rs;
  }
  if (ROWSUM) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      float v = rsum[c] + xor16f(rsum[c], lane);
      v += xor32f(v, lane);
      if (cv && qd == 0) {
        a.w.Dc[c * BTH + row] = gc[c] * v;
        a.w.dz[row * 3 + c] = v * gc[c] * (1.f - gc[c]);
      }
    }
    return;
  }
  if (cv) {
    float* out = a.dq + row * DK + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
      store4(out + dt * 16, dm.scale * st.dq[dt][0], dm.scale * st.dq[dt][1], dm.scale * st.dq[dt][2],
             dm.scale * st.dq[dt][3]);
  }
}

// ---------------------------------------------------------------------------
// dK / dV: one wave per 16 keys.
// ---------------------------------------------------------------------------
enum KvMode { KV_CMP = 0, KV_WIN = 1, KV_SLC = 2 };

template <typename T, int DK, int DV, int MODE>
__global__ __launch_bounds__(64) void k_bwd_kv(Dims dm, BwdArgs a) {
  const int lane = threadIdx.x, c16 = lane & 15, qd = lane >> 4;
  const BwdPlan& pl = a.pl;
  const int G = dm.G;
  const size_t BTH = (size_t)dm.B * dm.T * dm.Hq;
  int bg, k0, klim;            // keys k0 .. k0+15, valid below klim
  int p0 = 0, p1 = 0;          // position range (cmp, win)
  const int* plist = nullptr;  // position list (slc)
  int nlist = 0;
  float* outp = nullptr;       // partial output [16][DK+DV] (cmp, slc)
  int jblk = 0;
  if (MODE == KV_CMP) {
    const int seg = blockIdx.x % pl.nseg_cmp;
    const int r = blockIdx.x / pl.nseg_cmp;
    const int kt = r % pl.nkt_cmp;
    bg = r / pl.nkt_cmp;
    k0 = kt * 16;
    klim = dm.ncmp;
    const int pf = k0 * dm.d + dm.l - 1;
    p0 = pf + seg * kSegCmp;
    p1 = min(dm.T, p0 + kSegCmp);
    outp = a.w.part_cmp + ((size_t)blockIdx.x) * 16 * (DK + DV);
  } else if (MODE == KV_WIN) {
    const int ntk = (dm.T + 15) / 16;
    const int kt = blockIdx.x % ntk;
    bg = blockIdx.x / ntk;
    k0 = kt * 16;
    klim = dm.T;
    p0 = k0;
    p1 = min(dm.T, k0 + 15 + dm.w);
  } else {
    const int nsub = dm.ls / 16;
    const int seg = blockIdx.x % pl.nseg_slc;
    int r = blockIdx.x / pl.nseg_slc;
    const int sub = r % nsub;
    r /= nsub;
    jblk = r % dm.nsel;
    bg = r / dm.nsel;
    const int cnt = a.w.cnt[(size_t)bg * dm.nsel + jblk];
    if (seg * kSegSlc >= cnt) return;
    nlist = min(kSegSlc, cnt - seg * kSegSlc);
    plist = a.w.list + (size_t)bg * dm.T * dm.n + a.w.lstart[(size_t)bg * dm.nsel + jblk] + seg * kSegSlc;
    k0 = jblk * dm.ls + sub * 16;
    klim = min(dm.T, (jblk + 1) * dm.ls);
    const int slot = a.w.segoff[(size_t)bg * dm.nsel + jblk] + seg;
    outp = a.w.part_slc + ((size_t)bg * pl.max_slc_seg + slot) * dm.ls * (DK + DV) + (size_t)sub * 16 * (DK + DV);
  }
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int c = MODE == KV_CMP ? 0 : (MODE == KV_SLC ? 1 : 2);
  const int key = k0 + c16;   // this lane's key column
  const bool kvalid = key < klim;
  // B operands: K^T and V^T columns = this tile's 16 keys
  const T *kr, *vr;
  if (MODE == KV_CMP) {
    kr = (const T*)a.kc + ((size_t)(b * dm.ncmp + min(key, klim - 1)) * dm.Hkv + g) * DK;
    vr = (const T*)a.vc + ((size_t)(b * dm.ncmp + min(key, klim - 1)) * dm.Hkv + g) * DV;
  } else {
    kr = (const T*)a.k + ((size_t)(b * dm.T + min(key, klim - 1)) * dm.Hkv + g) * DK;
    vr = (const T*)a.v + ((size_t)(b * dm.T + min(key, klim - 1)) * dm.Hkv + g) * DV;
  }
  Frag8<T> kf[DK / 32], vf[DV / 32];
#pragma unroll
  for (int ks = 0; ks < DK / 32; ++ks) kf[ks] = load_frag(kr + ks * 32 + qd * 8);
#pragma unroll
  for (int ks = 0; ks < DV / 32; ++ks) vf[ks] = load_frag(vr + ks * 32 + qd * 8);
  f32x4 dk[DK / 16], dv[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DK / 16; ++dt) dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc2 = dm.scale * kLog2e;
  const T* qtb = (const T*)a.w.qt + (size_t)bg * DK * pl.Ts;
  const T* dotb = (const T*)a.w.dot + (size_t)bg * DV * pl.Ts;
  const int npos = (MODE == KV_SLC) ? nlist : max(0, p1 - p0);
  for (int pi = 0; pi < npos; pi += 2) {
    int pos[2];
    bool pv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      pv[i] = pi + i < npos;
      const int ii = pv[i] ? pi + i : pi;
      pos[i] = (MODE == KV_SLC) ? plist[ii] : p0 + ii;
    }
    float pg[2][4], dsv[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      // rows of this query tile: heads c16 (A operand) / 4qd + r (accumulator)
      const bool hv = c16 < G && pv[i];
      const size_t arow = (size_t)(b * dm.T + pos[i]) * dm.Hq + g * G + (c16 < G ? c16 : 0);
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
      const T* qp = (const T*)a.q + arow * DK + qd * 8;
      const T* dp_ = (const T*)a.d_o + arow * DV + qd * 8;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) mma(s, hv ? load_frag(qp + ks * 32) : zero_frag<T>(), kf[ks]);
#pragma unroll
      for (int ks = 0; ks < DV / 32; ++ks) mma(dp, hv ? load_frag(dp_ + ks * 32) : zero_frag<T>(), vf[ks]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hh = qd * 4 + r;
        bool v = hh < G && pv[i] && kvalid;
        const int t = pos[i];
        if (MODE == KV_CMP) v = v && key < ncmp_visible(t, dm.l, dm.d);
        else if (MODE == KV_WIN) v = v && key <= t && t <= key + dm.w - 1;
        else v = v && key <= t;
        const size_t rr = (size_t)(b * dm.T + t) * dm.Hq + g * G + (hh < G ? hh : 0);
        float p = 0.f, ds = 0.f;
        if (v) {
          const float gcv = a.w.gates[rr * 3 + c];
          p = fast_exp2(s[r] * sc2 - a.lse[c * BTH + rr] * kLog2e);
          ds = p * (gcv * dp[r] - a.w.Dc[c * BTH + rr]);
          p *= gcv;
        }
        pg[i][r] = p;
        dsv[i][r] = ds;
      }
    }
    float pv8[8], ds8[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pv8[e] = pg[0][e]; pv8[4 + e] = pg[1][e];
      ds8[e] = dsv[0][e]; ds8[4 + e] = dsv[1][e];
    }
    // P and dS enter sums over up to T*G query rows: carry them as bf16 hi + lo
    // pairs (about 16 significant bits) so the key gradients stay accurate.
    Frag8<T> pfr = to_frag<T>(pv8), dsf = to_frag<T>(ds8), plo, dslo;
    if constexpr (sizeof(T) == 2) {
      split_bf16(pv8, pfr, plo);
      split_bf16(ds8, dsf, dslo);
    }
    // A operands from the transposed q / dO: row = feature, k = (position, head) pairs
    const size_t f0 = (size_t)pos[0] * 16 + qd * 4, f1 = (size_t)pos[1] * 16 + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      const T* src = dotb + (size_t)(dt * 16 + c16) * pl.Ts;
      float x[8];
      load4(src + f0, x);
      load4(src + f1, x + 4);
      const Frag8<T> xf = to_frag<T>(x);
      mma(dv[dt], xf, pfr);
      if constexpr (sizeof(T) == 2) mma(dv[dt], xf, plo);
    }
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      const T* src = qtb + (size_t)(dt * 16 + c16) * pl.Ts;
      float x[8];
      load4(src + f0, x);
      load4(src + f1, x + 4);
      const Frag8<T> xf = to_frag<T>(x);
      mma(dk[dt], xf, dsf);
      if constexpr (sizeof(T) == 2) mma(dk[dt], xf, dslo);
    }
  }
  // write: lane holds key column c16, features dt*16 + 4qd + r
  if (MODE == KV_WIN) {
    if (!kvalid) return;
    float* dkp = a.dk + ((size_t)(b * dm.T + key) * dm.Hkv + g) * DK + qd * 4;
    float* dvp = a.dv + ((size_t)(b * dm.T + key) * dm.Hkv + g) * DV + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
      store4(dkp + dt * 16, dm.scale * dk[dt][0], dm.scale * dk[dt][1], dm.scale * dk[dt][2], dm.scale * dk[dt][3]);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) store4(dvp + dt * 16, dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]);
  } else {
    float* op = outp + (size_t)c16 * (DK + DV) + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
      store4(op + dt * 16, dm.scale * dk[dt][0], dm.scale * dk[dt][1], dm.scale * dk[dt][2], dm.scale * dk[dt][3]);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) store4(op + DK + dt * 16, dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]);
  }
}

// Sum the compressed-key segments in order: dkc/dvc [B,Hkv,ncmp,D].
__global__ __launch_bounds__(256) void k_reduce_cmp(Dims dm, BwdArgs a) {
  const BwdPlan& pl = a.pl;
  const int W = dm.dk + dm.dv;
  const int r = blockIdx.x;              // (bg, kt)
  const int kt = r % pl.nkt_cmp, bg = r / pl.nkt_cmp;
  for (int i = threadIdx.x; i < 16 * W; i += 256) {
    const int kk = i / W, e = i % W, key = kt * 16 + kk;
    if (key >= dm.ncmp) continue;
    // segments of this key tile start at its first visible position
    const int pf = (kt * 16) * dm.d + dm.l - 1;
    float s = 0.f;
    for (int seg = 0; seg < pl.nseg_cmp; ++seg) {
      if (pf + seg * kSegCmp >= dm.T) break;
      s += a.w.part_cmp[(((size_t)r * pl.nseg_cmp + seg) * 16 + kk) * W + e];
    }
    if (e < dm.dk) a.w.dkc[((size_t)bg * dm.ncmp + key) * dm.dk + e] = s;
    else a.w.dvc[((size_t)bg * dm.ncmp + key) * dm.dv + e - dm.dk] = s;
  }
}

// Add the selected-block segments, in order, into dk / dv.
__global__ __launch_bounds__(256) void k_reduce_slc(Dims dm, BwdArgs a) {
  const BwdPlan& pl = a.pl;
  const int W = dm.dk + dm.dv;
  const int j = blockIdx.x % dm.nsel, bg = blockIdx.x / dm.nsel;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int cnt = a.w.cnt[(size_t)bg * dm.nsel + j];
  if (cnt == 0) return;
  const int nseg = (cnt + kSegSlc - 1) / kSegSlc;
  const int slot0 = a.w.segoff[(size_t)bg * dm.nsel + j];
  for (int i = threadIdx.x; i < dm.ls * W; i += 256) {
    const int kk = i / W, e = i % W, key = j * dm.ls + kk;
    if (key >= dm.T) continue;
    float s = 0.f;
    for (int sg = 0; sg < nseg; ++sg)
      s += a.w.part_slc[(((size_t)bg * pl.max_slc_seg + slot0 + sg) * dm.ls + kk) * W + e];
    if (e < dm.dk) a.dk[((size_t)(b * dm.T + key) * dm.Hkv + g) * dm.dk + e] += s;
    else a.dv[((size_t)(b * dm.T + key) * dm.Hkv + g) * dm.dv + e - dm.dk] += s;
  }
}

// ---------------------------------------------------------------------------
// Reverse index: positions that selected each block, ascending.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_rev_hist(Dims dm, BwdArgs a) {
  extern __shared__ int hist[];
  const BwdPlan& pl = a.pl;
  const int ch = blockIdx.x % pl.nchunk, bg = blockIdx.x / pl.nchunk;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  for (int j = threadIdx.x; j < dm.nsel; j += 64) hist[j] = 0;
  __syncthreads();
  const int t0 = ch * kRevChunk, t1 = min(dm.T, t0 + kRevChunk);
  for (int t = t0; t < t1; ++t) {
    if (threadIdx.x < dm.n) {
      const int j = a.idx[((size_t)(b * dm.T + t) * dm.Hkv + g) * dm.n + threadIdx.x];
      if (j >= 0) hist[j] += 1;
    }
    __syncthreads();
  }
  for (int j = threadIdx.x; j < dm.nsel; j += 64)
    a.w.hist[((size_t)bg * pl.nchunk + ch) * dm.nsel + j] = hist[j];
}

__global__ __launch_bounds__(256) void k_rev_scan(Dims dm, BwdArgs a) {
  const BwdPlan& pl = a.pl;
  const int bg = blockIdx.x;
  for (int j = threadIdx.x; j < dm.nsel; j += 256) {
    int tot = 0;
    for (int ch = 0; ch < pl.nchunk; ++ch) tot += a.w.hist[((size_t)bg * pl.nchunk + ch) * dm.nsel + j];
    a.w.cnt[(size_t)bg * dm.nsel + j] = tot;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0, srun = 0;
    for (int j = 0; j < dm.nsel; ++j) {
      const int c = a.w.cnt[(size_t)bg * dm.nsel + j];
      a.w.lstart[(size_t)bg * dm.nsel + j] = run;
      a.w.segoff[(size_t)bg * dm.nsel + j] = srun;
      run += c;
      srun += (c + kSegSlc - 1) / kSegSlc;
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < dm.nsel; j += 256) {
    int run = a.w.lstart[(size_t)bg * dm.nsel + j];
    for (int ch = 0; ch < pl.nchunk; ++ch) {
      const size_t o = ((size_t)bg * pl.nchunk + ch) * dm.nsel + j;
      a.w.offc[o] = run;
      run += a.w.hist[o];
    }
  }
}

__global__ __launch_bounds__(64) void k_rev_fill(Dims dm, BwdArgs a) {
  extern __shared__ int cur[];
  const BwdPlan& pl = a.pl;
  const int ch = blockIdx.x % pl.nchunk, bg = blockIdx.x / pl.nchunk;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  for (int j = threadIdx.x; j < dm.nsel; j += 64) cur[j] = a.w.offc[((size_t)bg * pl.nchunk + ch) * dm.nsel + j];
  __syncthreads();
  int* list = a.w.list + (size_t)bg * dm.T * dm.n;
  const int t0 = ch * kRevChunk, t1 = min(dm.T, t0 + kRevChunk);
  for (int t = t0; t < t1; ++t) {
    if (threadIdx.x < dm.n) {
      const int j = a.idx[((size_t)(b * dm.T + t) * dm.Hkv + g) * dm.n + threadIdx.x];
      if (j >= 0) list[cur[j]++] = t;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Strided fp32 GEMM on MFMA: C[m,n] (+)= sum_k A[m*sam + k*sak] * B[k*sbk + n*sbn].
// 64x64 output tile per workgroup, k steps of 32 staged through LDS.
// ---------------------------------------------------------------------------
struct Gemm {
  int M, N, K;
  const void* A; long long sam, sak;
  const void* B; long long sbk, sbn;
  float* C; long long ldc;
  int accumulate;
};

template <typename TA, typename TB>
__global__ __launch_bounds__(256) void k_gemm(Gemm gm) {
  __shared__ float As[32][64 + 4];
  __shared__ float Bs[32][64 + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kq = lane >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const TA* A = (const TA*)gm.A;
  const TB* B = (const TB*)gm.B;
  f32x4 acc[2][2];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool a_k_fast = gm.sak == 1, b_n_fast = gm.sbn == 1;
  for (int k0 = 0; k0 < gm.K; k0 += 32) {
    for (int i = tid; i < 64 * 32; i += 256) {
      int mm, kk;
      if (a_k_fast) { kk = i & 31; mm = i >> 5; } else { mm = i & 63; kk = i >> 6; }
      const int m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < gm.M && k < gm.K) ? to_f32(A[m * gm.sam + k * gm.sak]) : 0.f;
      int nn, kb;
      if (b_n_fast) { nn = i & 63; kb = i >> 6; } else { kb = i & 31; nn = i >> 5; }
      const int n = n0 + nn, k2 = k0 + kb;
      Bs[kb][nn] = (n < gm.N && k2 < gm.K) ? to_f32(B[k2 * gm.sbk + n * gm.sbn]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 32; kk += 4) {
      float af[2], bfv[2];
      for (int i = 0; i < 2; ++i) af[i] = As[kk + kq][(wave >> 1) * 32 + i * 16 + c16];
      for (int j = 0; j < 2; ++j) bfv[j] = Bs[kk + kq][(wave & 1) * 32 + j * 16 + c16];
      for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bfv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + (wave & 1) * 32 + j * 16 + c16;
      if (n >= gm.N) continue;
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + (wave >> 1) * 32 + i * 16 + kq * 4 + r;
        if (m >= gm.M) continue;
        float* cp = gm.C + (long long)m * gm.ldc + n;
        *cp = gm.accumulate ? *cp + acc[i][j][r] : acc[i][j][r];
      }
    }
}

template <typename TA, typename TB>
static hipError_t gemm(const Gemm& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  dim3 grid((g.N + 63) / 64, (g.M + 63) / 64);
  k_gemm<TA, TB><<<grid, 256, 0, s>>>(g);
  return hipGetLastError();
}

// Column sums: out[c] (+)= sum_r in[r*ld + c].  Fixed order per column.
__global__ __launch_bounds__(256) void k_colsum(int R, int Cn, long long ld, const float* __restrict__ in,
                                                float* __restrict__ out, int accumulate) {
  __shared__ float part[4][64];
  const int c = blockIdx.x * 64 + (threadIdx.x & 63), rg = threadIdx.x >> 6;
  float s = 0.f;
  if (c < Cn)
    for (int r = rg; r < R; r += 4) s += in[(long long)r * ld + c];
  part[rg][threadIdx.x & 63] = s;
  __syncthreads();
  if (rg == 0 && c < Cn) {
    const float v = part[0][threadIdx.x] + part[1][threadIdx.x] + part[2][threadIdx.x] + part[3][threadIdx.x];
    out[c] = accumulate ? out[c] + v : v;
  }
}

// ---------------------------------------------------------------------------
// phi backward.
// ---------------------------------------------------------------------------
// Pre-activation a and gelu(a) from the sub-block products y (see the forward).
template <typename T>
__global__ __launch_bounds__(256) void k_phi_act(Dims dm, const float* __restrict__ y, const T* __restrict__ b1,
                                                 float* __restrict__ act, float* __restrict__ hid) {
  const int H = dm.hidden, R = dm.l / dm.d, N = R * H;
  const int nsub = dm.ncmp + R - 1;
  const size_t rows = (size_t)dm.B * dm.Hkv * dm.ncmp;
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * H) return;
  const int o = id % H;
  const size_t row = id / H;
  const int i = row % dm.ncmp;
  const size_t bg = row / dm.ncmp;
  const size_t Mmain = (size_t)dm.B * dm.Hkv * nsub;
  float v = to_f32(b1[o]);
  for (int r = 0; r < R; ++r) v += y[(Mmain + r) * N + (size_t)r * H + o];
  for (int r = 0; r < R; ++r) v += y[(bg * nsub + i + r) * N + (size_t)r * H + o];
  act[id] = v;
  hid[id] = 0.5f * v * (1.f + erff(v * 0.70710678118654752f));
}

__global__ __launch_bounds__(256) void k_phi_dact(size_t n, const float* __restrict__ act, float* __restrict__ dh) {
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= n) return;
  const float a = act[id];
  const float cdf = 0.5f * (1.f + erff(a * 0.70710678118654752f));
  const float pdf = 0.3989422804014327f * expf(-0.5f * a * a);
  dh[id] *= cdf + a * pdf;
}

// dW1[r*d*D + x][o] = sum_{bg,i} (x_tok[bg, (i+r)*d + j][e] + pe[r*d + j][e]) * da[(bg,i)][o],
// x = j*D + e.  64 x 64 output tile per workgroup, rows in steps of 32.
template <typename T>
__global__ __launch_bounds__(256) void k_phi_dw1(Dims dm, int D, const T* __restrict__ xs, const T* __restrict__ pe,
                                                 const float* __restrict__ da, float* __restrict__ dw1) {
  __shared__ float As[32][64 + 4];
  __shared__ float Bs[32][64 + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kq = lane >> 4;
  const int H = dm.hidden, dD = dm.d * D;
  const int r = blockIdx.z;
  const int x0 = blockIdx.y * 64, o0 = blockIdx.x * 64;
  const int rows = dm.B * dm.Hkv * dm.ncmp;
  f32x4 acc[2][2];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < rows; k0 += 32) {
    for (int i = tid; i < 64 * 32; i += 256) {
      const int xx = i & 63, kk = i >> 6, row = k0 + kk, xg = x0 + xx;
      float v = 0.f;
      if (row < rows && xg < dD) {
        const int ii = row % dm.ncmp, bg = row / dm.ncmp, b = bg / dm.Hkv, g = bg % dm.Hkv;
        const int j = xg / D, e = xg % D;
        const int tok = (ii + r) * dm.d + j;
        v = to_f32(xs[((size_t)(b * dm.T + tok) * dm.Hkv + g) * D + e]) + to_f32(pe[(size_t)(r * dm.d + j) * D + e]);
      }
      As[kk][xx] = v;
      const int oo = i & 63, o = o0 + oo;
      Bs[kk][oo] = (row < rows && o < H) ? da[(size_t)row * H + o] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 32; kk += 4) {
      float af[2], bfv[2];
      for (int i = 0; i < 2; ++i) af[i] = As[kk + kq][(wave >> 1) * 32 + i * 16 + c16];
      for (int j = 0; j < 2; ++j) bfv[j] = Bs[kk + kq][(wave & 1) * 32 + j * 16 + c16];
      for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bfv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) {
      const int o = o0 + (wave & 1) * 32 + j * 16 + c16;
      for (int rr = 0; rr < 4; ++rr) {
        const int xg = x0 + (wave >> 1) * 32 + i * 16 + kq * 4 + rr;
        if (xg < dD && o < H) dw1[((size_t)r * dD + xg) * H + o] = acc[i][j][rr];
      }
    }
}

// Token gradient from phi: dx[b, tok, g, e] += sum over blocks i covering tok of
// du[(bg, i)][(tok - i*d)*D + e]   (MLP), or of dcmp[(bg,i)][e] / l (mean).
__global__ __launch_bounds__(256) void k_phi_dx(Dims dm, int D, const float* __restrict__ src, int mlp,
                                                float* __restrict__ dx) {
  const size_t total = (size_t)dm.B * dm.T * dm.Hkv * D;
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= total) return;
  const int e = id % D;
  size_t r = id / D;
  const int g = r % dm.Hkv;
  r /= dm.Hkv;
  const int tok = r % dm.T, b = r / dm.T;
  const int bg = b * dm.Hkv + g;
  // blocks i with i*d <= tok < i*d + l, 0 <= i < ncmp
  int ilo = tok - dm.l + 1;
  ilo = ilo <= 0 ? 0 : (ilo + dm.d - 1) / dm.d;
  const int ihi = min(tok / dm.d, dm.ncmp - 1);
  float s = 0.f;
  for (int i = ilo; i <= ihi; ++i) {
    const size_t row = (size_t)bg * dm.ncmp + i;
    if (mlp) s += src[row * dm.l * D + (size_t)(tok - i * dm.d) * D + e];
    else s += src[row * D + e] / (float)dm.l;
  }
  dx[id] += s;
}

template <typename T, int D>
static hipError_t phi_bwd(const Dims& dm, const BwdArgs& a, const nsa_phi_weights& w, const nsa_phi_grads& gr,
                          const void* xsrc, const float* dcmp, float* dx, hipStream_t s) {
  hipError_t e;
  const size_t rows = (size_t)dm.B * dm.Hkv * dm.ncmp;
  if (dm.hidden == 0) {
    if (dm.ncmp == 0) return hipSuccess;
    const size_t total = (size_t)dm.B * dm.T * dm.Hkv * D;
    k_phi_dx<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(dm, D, dcmp, 0, dx);
    return hipGetLastError();
  }
  const int H = dm.hidden, R = dm.l / dm.d;
  const int nsub = dm.ncmp + R - 1;
  // recompute the forward pre-activations
  if ((e = launch_transpose_2d(dm, dm.l * D, H, w.w1, a.w.w1t, s)) != hipSuccess) return e;
  if ((e = launch_phi_gemm1(dm, D, nsub, xsrc, w.pe, a.w.w1t, a.w.y, s)) != hipSuccess) return e;
  k_phi_act<T><<<(unsigned)((rows * H + 255) / 256), 256, 0, s>>>(dm, a.w.y, (const T*)w.b1, a.w.act, a.w.hid);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // db2 = colsum(dout); dW2 = hid^T dout
  k_colsum<<<(D + 63) / 64, 256, 0, s>>>((int)rows, D, D, dcmp, (float*)gr.b2, 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    Gemm g{H, D, (int)rows, a.w.hid, 1, H, dcmp, D, 1, (float*)gr.w2, D, 0};
    if ((e = gemm<float, float>(g, s)) != hipSuccess) return e;
  }
  // dh = dout W2^T; da = dh * gelu'(act)
  {
    Gemm g{(int)rows, H, D, dcmp, D, 1, w.w2, 1, D, a.w.dh, H, 0};
    if ((e = gemm<float, T>(g, s)) != hipSuccess) return e;
  }
  k_phi_dact<<<(unsigned)((rows * H + 255) / 256), 256, 0, s>>>(rows * H, a.w.act, a.w.dh);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_colsum<<<(H + 63) / 64, 256, 0, s>>>((int)rows, H, H, a.w.dh, (float*)gr.b1, 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dW1 chunks
  {
    dim3 grid((H + 63) / 64, (dm.d * D + 63) / 64, R);
    k_phi_dw1<T><<<grid, 256, 0, s>>>(dm, D, (const T*)xsrc, (const T*)w.pe, a.w.dh, (float*)gr.w1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // du = da W1^T -> token gradient and dpe
  {
    Gemm g{(int)rows, dm.l * D, H, a.w.dh, H, 1, w.w1, 1, H, a.w.du, (long long)dm.l * D, 0};
    if ((e = gemm<float, T>(g, s)) != hipSuccess) return e;
  }
  k_colsum<<<(dm.l * D + 63) / 64, 256, 0, s>>>((int)rows, dm.l * D, (long long)dm.l * D, a.w.du, (float*)gr.pe, 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t total = (size_t)dm.B * dm.T * dm.Hkv * D;
  k_phi_dx<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(dm, D, a.w.du, 1, dx);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_fill_f32(size_t n, float* __restrict__ p) {
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id < n) p[id] = 0.f;
}

static hipError_t zero_f32(float* p, size_t n, hipStream_t s) {
  if (!n) return hipSuccess;
  k_fill_f32<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(n, p);
  return hipGetLastError();
}

template <typename T, int DK, int DV>
static hipError_t bwd_impl(const Dims& dm, const nsa_bwd_args* args, BwdArgs& a, hipStream_t s, void* const* events) {
  int ei = 0;
  auto mark = [&]() { return events ? hipEventRecord((hipEvent_t)events[ei++], s) : hipSuccess; };
  hipError_t e;
  const BwdPlan& pl = a.pl;
  const size_t BTH = (size_t)dm.B * dm.T * dm.Hq;
  const int BG = dm.B * dm.Hkv;
  // stage 0: gates, gate backward, row terms
  if ((e = mark()) != hipSuccess) return e;
  if ((e = launch_gate(dm, dm.B * dm.T, a.x, a.wg, a.w.gates, s)) != hipSuccess) return e;
  // stage 1: transposed copies
  if ((e = mark()) != hipSuccess) return e;
  if ((e = launch_transpose_seq(dm, dm.B, dm.T, dm.Hkv, DK, dm.Tp, a.k, a.w.kt, s)) != hipSuccess) return e;
  if (dm.ncmp > 0 &&
      (e = launch_transpose_seq(dm, dm.B, dm.ncmp, dm.Hkv, DK, dm.ncmp_pad, a.kc, a.w.kct, s)) != hipSuccess)
    return e;
  {
    dim3 gq((pl.Ts + 63) / 64, (DK + 63) / 64, BG), gd((pl.Ts + 63) / 64, (DV + 63) / 64, BG);
    k_transpose_heads<T><<<gq, 256, 0, s>>>(dm, DK, (const T*)a.q, (T*)a.w.qt);
    k_transpose_heads<T><<<gd, 256, 0, s>>>(dm, DV, (const T*)a.d_o, (T*)a.w.dot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // stage 2: row terms D_c, dz, then dq
  if ((e = mark()) != hipSuccess) return e;
  k_bwd_dq<T, DK, DV, true><<<((dm.T + 3) / 4) * BG, 256, 0, s>>>(dm, a);
  k_bwd_dq<T, DK, DV, false><<<((dm.T + 3) / 4) * BG, 256, 0, s>>>(dm, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // stage 3: compressed keys
  if ((e = mark()) != hipSuccess) return e;
  if (dm.ncmp > 0) {
    k_bwd_kv<T, DK, DV, KV_CMP><<<BG * pl.nkt_cmp * pl.nseg_cmp, 64, 0, s>>>(dm, a);
    k_reduce_cmp<<<BG * pl.nkt_cmp, 256, 0, s>>>(dm, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // stage 4: window keys (writes dk, dv)
  if ((e = mark()) != hipSuccess) return e;
  k_bwd_kv<T, DK, DV, KV_WIN><<<BG * ((dm.T + 15) / 16), 64, 0, s>>>(dm, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // stage 5: selected blocks (adds into dk, dv)
  if ((e = mark()) != hipSuccess) return e;
  k_rev_hist<<<BG * pl.nchunk, 64, dm.nsel * sizeof(int), s>>>(dm, a);
  k_rev_scan<<<BG, 256, 0, s>>>(dm, a);
  k_rev_fill<<<BG * pl.nchunk, 64, dm.nsel * sizeof(int), s>>>(dm, a);
  k_bwd_kv<T, DK, DV, KV_SLC><<<BG * dm.nsel * (dm.ls / 16) * pl.nseg_slc, 64, 0, s>>>(dm, a);
  k_reduce_slc<<<BG * dm.nsel, 256, 0, s>>>(dm, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // stage 6: phi
  if ((e = mark()) != hipSuccess) return e;
  if (dm.hidden && dm.ncmp == 0) {
    const nsa_phi_grads* gs[2] = {&args->d_phi_k, &args->d_phi_v};
    const int Ds[2] = {DK, DV};
    for (int t = 0; t < 2; ++t) {
      if ((e = zero_f32((float*)gs[t]->pe, (size_t)dm.l * Ds[t], s)) != hipSuccess) return e;
      if ((e = zero_f32((float*)gs[t]->w1, (size_t)dm.l * Ds[t] * dm.hidden, s)) != hipSuccess) return e;
      if ((e = zero_f32((float*)gs[t]->b1, (size_t)dm.hidden, s)) != hipSuccess) return e;
      if ((e = zero_f32((float*)gs[t]->w2, (size_t)dm.hidden * Ds[t], s)) != hipSuccess) return e;
      if ((e = zero_f32((float*)gs[t]->b2, (size_t)Ds[t], s)) != hipSuccess) return e;
    }
  } else {
    if ((e = phi_bwd<T, DK>(dm, a, args->phi_k, args->d_phi_k, a.k, a.w.dkc, a.dk, s)) != hipSuccess) return e;
    if ((e = phi_bwd<T, DV>(dm, a, args->phi_v, args->d_phi_v, a.v, a.w.dvc, a.dv, s)) != hipSuccess) return e;
  }
  // stage 7: dW_g = x^T dz
  if ((e = mark()) != hipSuccess) return e;
  {
    Gemm g{dm.C, 3 * dm.Hq, dm.B * dm.T, a.x, 1, dm.C, a.w.dz, 3 * dm.Hq, 1, a.dwg, 3 * dm.Hq, 0};
    if ((e = gemm<T, float>(g, s)) != hipSuccess) return e;
  }
  return mark();
}

hipError_t launch_bwd(const Dims& dm, const nsa_bwd_args* args, void* ws, hipStream_t s, void* const* events) {
  BwdArgs a;
  a.q = args->q; a.k = args->k; a.v = args->v; a.x = args->x; a.wg = args->w_gate;
  a.kc = args->k_cmp; a.vc = args->v_cmp; a.d_o = args->d_o;
  a.lse = (const float*)args->lse; a.idx = (const int*)args->idx;
  a.dq = (float*)args->dq; a.dk = (float*)args->dk; a.dv = (float*)args->dv; a.dwg = (float*)args->dw_gate;
  bwd_carve(dm, ws, &a.w);
  a.pl = bwd_plan(dm);
  const bool bf = dm.io == IO_BF16;
  if (dm.dk == 64 && dm.dv == 64) return bf ? bwd_impl<bf16, 64, 64>(dm, args, a, s, events) : bwd_impl<float, 64, 64>(dm, args, a, s, events);
  if (dm.dk == 128 && dm.dv == 128) return bf ? bwd_impl<bf16, 128, 128>(dm, args, a, s, events) : bwd_impl<float, 128, 128>(dm, args, a, s, events);
  if (dm.dk == 192 && dm.dv == 128) return bf ? bwd_impl<bf16, 192, 128>(dm, args, a, s, events) : bwd_impl<float, 192, 128>(dm, args, a, s, events);
  return hipErrorInvalidValue;
}

}  // namespace nsa
