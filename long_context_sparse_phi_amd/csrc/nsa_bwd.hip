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
//   * phi's first layer: recomputed with the bf16 MFMA GEMM; its weight and
//     token gradients are the same GEMM over the sub-block rows (da shifted
//     into the same row layout, see phi_bwd).  phi's second layer and the
//     gate projection go through the strided fp32 MFMA GEMM.
#include <type_traits>

#include "../../include/nsa.h"
#include "nsa_common.hpp"
#include "nsa_kernels.hpp"

namespace nsa {

int bwd_stage_count() { return 8; }

constexpr int kSegCmp = 512;     // query positions per compressed-key segment
constexpr int kSegSlc = 512;     // list entries per selected-block segment
constexpr int kRevChunk = 256;   // positions per reverse-index chunk
constexpr int kMaxSplit = 64;    // split-K factor bound of the reduction GEMMs
constexpr int kW1Split = 16;     // split-K factor bound of phi's dW1 GEMM (bf16 I/O)

struct BwdPlan {
  int nkg_cmp;     // 64-key groups of the compressed keys
  int nseg_cmp;    // position segments per compressed key group (upper bound)
  int nchunk;      // reverse-index chunks
  int nkc_slc;     // 64-key chunks per selection block
  int nseg_slc;    // segments per selected block (upper bound)
  int max_slc_seg; // segment slots per (b, g)
};

static BwdPlan bwd_plan(const Dims& dm) {
  BwdPlan p;
  p.nkg_cmp = (dm.ncmp + 63) / 64;
  p.nseg_cmp = (dm.T + kSegCmp - 1) / kSegCmp;
  p.nchunk = (dm.T + kRevChunk - 1) / kRevChunk;
  p.nkc_slc = (dm.ls + 63) / 64;
  p.nseg_slc = (dm.T + kSegSlc - 1) / kSegSlc;
  p.max_slc_seg = dm.nsel + (int)(((long long)dm.T * dm.n + kSegSlc - 1) / kSegSlc);
  return p;
}

struct BwdBufs {
  float* gates;    // [B,T,Hq,3]
  float* ghid;     // gate MLP: hidden layer gelu(x w1 + b1) [B*T, Cg]
  float* gpre;     // gate MLP: the same before the GELU
  float* gdh;      // gate MLP: gradient of the hidden layer [B*T, Cg]
  float* Dc;       // [3,B,T,Hq]
  float* dz;       // [B,T,Hq,3]
  void* fkv;       // fragment tiles of (k, v, k^T) over T (bwd_tile_ins instructions per 32 keys)
                   // of the selected branch's keys/values
  void* fkvw;      // the same for the window branch's own keys/values (independent K/V only)
  void* fckv;      // the same over the compressed keys (k_cmp, v_cmp, k_cmp^T)
  float* dkc;      // [B,Hkv,ncmp,dk]
  float* dvc;      // [B,Hkv,ncmp,dv]
  float* part_cmp; // [B*Hkv*nkg*nseg][64][dk+dv]
  int* hist;       // [B*Hkv][nchunk][nsel]
  int* offc;       // [B*Hkv][nchunk][nsel]
  int* cnt;        // [B*Hkv][nsel]
  int* lstart;     // [B*Hkv][nsel]
  int* segoff;     // [B*Hkv][nsel]
  int* task;       // [B*Hkv][max_slc_seg] segment slot -> j * nseg_slc + seg, or -1
  int* list;       // [B*Hkv][T*n]
  float* part_slc; // [B*Hkv*max_slc_seg][ls][dk+dv]
  float* gpart;    // split-K GEMM / column-sum partials
  // phi
  void* arows;     // [B*Hkv*nsub + l/d, d*D] io: phi GEMM1 rows
  void* w2t;       // [D, H]     io
  float* y;        // GEMM1 output
  float* act;      // [rows,H] pre-activation (rows = B*Hkv*ncmp compressed keys)
  float* hid;      // [rows,H] gelu(act)
  float* dh;       // [rows,H]
  float* dap;      // [B*Hkv*nsub + l/d - 1, H] dh * gelu'(act) in the sub-block row layout
  float* dxs;      // [B*Hkv*nsub, d*D] token gradient of phi per sub-block
  float* pe_part;  // position-embedding rows' partial sums (launch_phi_gemm1)
};

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Fragment tile of the dq passes: key-row fragments of k (2*dk/32) and of v
// (2*dv/32), then transposed fragments of k (dk/16).
static int bwd_tile_ins(const Dims& dm) { return 2 * dm.dk / 32 + 2 * dm.dv / 32 + dm.dk / 16; }

static size_t bwd_carve(const Dims& dm, void* ws, BwdBufs* w) {
  const BwdPlan p = bwd_plan(dm);
  char* base = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t bytes) { void* r = base ? base + off : nullptr; off += al256(bytes); return r; };
  const size_t es = dm.io == IO_BF16 ? 2 : 4;
  const size_t BTH = (size_t)dm.B * dm.T * dm.Hq, BG = (size_t)dm.B * dm.Hkv;
  w->gates = (float*)take(BTH * 3 * 4);
  w->ghid = (float*)take((size_t)dm.B * dm.T * dm.Cg * 4);
  w->gpre = (float*)take((size_t)dm.B * dm.T * dm.Cg * 4);
  w->gdh = (float*)take((size_t)dm.B * dm.T * dm.Cg * 4);
  w->Dc = (float*)take(3 * BTH * 4);
  w->dz = (float*)take(BTH * 3 * 4);
  w->fkv = take(frag_tiles_elems(dm, dm.T, bwd_tile_ins(dm)) * es);
  w->fkvw = take(frag_tiles_elems(dm, dm.T, bwd_tile_ins(dm)) * es);
  w->fckv = take(frag_tiles_elems(dm, dm.ncmp, bwd_tile_ins(dm)) * es);
  w->dkc = (float*)take(BG * dm.ncmp * dm.dk * 4);
  w->dvc = (float*)take(BG * dm.ncmp * dm.dv * 4);
  w->part_cmp = (float*)take(BG * p.nkg_cmp * p.nseg_cmp * 64 * (dm.dk + dm.dv) * 4);
  w->hist = (int*)take(BG * p.nchunk * dm.nsel * 4);
  w->offc = (int*)take(BG * p.nchunk * dm.nsel * 4);
  w->cnt = (int*)take(BG * dm.nsel * 4);
  w->lstart = (int*)take(BG * dm.nsel * 4);
  w->segoff = (int*)take(BG * dm.nsel * 4);
  w->task = (int*)take(BG * p.max_slc_seg * 4);
  w->list = (int*)take(BG * dm.T * dm.n * 4);
  w->part_slc = (float*)take(BG * p.max_slc_seg * dm.ls * (dm.dk + dm.dv) * 4);
  {
    const size_t Dm = dm.dk > dm.dv ? dm.dk : dm.dv;
    size_t mn = (size_t)dm.C * 3 * dm.Hq;
    mn = mn > (size_t)dm.hidden * Dm ? mn : (size_t)dm.hidden * Dm;
    mn = mn > (size_t)dm.l * Dm ? mn : (size_t)dm.l * Dm;
    mn = mn > (size_t)dm.Cg * 3 * dm.Hq ? mn : (size_t)dm.Cg * 3 * dm.Hq;
    mn = mn > (size_t)dm.C * dm.Cg ? mn : (size_t)dm.C * dm.Cg;
    // phi's dW1 chunks (d*D x hidden), split over the sub-block rows
    const size_t w1 = (size_t)dm.d * Dm * dm.hidden * (dm.io == IO_BF16 ? kW1Split : kGemmMaxSplit);
    w->gpart = (float*)take((kMaxSplit * mn > w1 ? kMaxSplit * mn : w1) * 4);
  }
  if (dm.hidden) {
    const int D = dm.dk > dm.dv ? dm.dk : dm.dv;
    const int R = dm.l / dm.d;
    const size_t rows = BG * dm.ncmp;
    const size_t nsub = dm.ncmp > 0 ? dm.ncmp + R - 1 : 0;
    w->arows = take((BG * nsub + R) * dm.d * D * es);
    w->w2t = take((size_t)D * dm.hidden * es);
    w->y = (float*)take((BG * nsub + R) * R * dm.hidden * 4);
    w->pe_part = (float*)take(phi_pe_part_floats(dm) * 4);
    w->act = (float*)take(rows * dm.hidden * 4);
    w->hid = (float*)take(rows * dm.hidden * 4);
    w->dh = (float*)take(rows * dm.hidden * 4);
    w->dap = (float*)take((nsub ? BG * nsub + R - 1 : 0) * dm.hidden * 4);
    w->dxs = (float*)take(BG * nsub * dm.d * D * 4);
  }
  return off;
}

size_t bwd_ws_bytes(const Dims& dm) {
  BwdBufs w;
  return bwd_carve(dm, nullptr, &w);
}

// k, v feed phi (the compressed branch); ks, vs the selected and kw, vw the
// window branch (all three the same tensors unless each branch has its own).
// dk, dv receive the phi path, dks/dvs and dkw/dvw the other two branches'
// key/value gradients (aliases of dk, dv when the tensors are shared).
struct BwdArgs {
  const void *q, *k, *v, *x, *wg, *kc, *vc, *d_o;
  const void *ks, *vs, *kw, *vw;
  const void* fkv_win;  // fragment tiles the dq pass reads for the window branch
  const float* ob;   // optional [3,B,T,Hq,dv] fp32 branch outputs saved by the forward
  const float* lse;  // [3,B,T,Hq] natural log
  const int* idx;    // [B,T,Hkv,n]
  float *dq, *dk, *dv, *dwg;
  float *dks, *dvs, *dkw, *dvw;
  bool split;
  BwdBufs w;
  BwdPlan pl;
};

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

// One 32-key tile of one branch.  tb: the packed fragment tile of keys
// kt .. kt+31 (already offset by lane*8); keys lo <= key < hi are valid.
// ROWSUM: accumulate sum_k P_k dP_k (dP = dO v^T, no gate), which equals
// <dO, O_c> exactly; otherwise accumulate dq^T += K^T dS^T.
template <typename T, int DK, int DV, bool ROWSUM>
__device__ __forceinline__ void dq_tile(DqState<T, DK, DV>& st, const T* tb, int kt, int lo, int hi, int c16,
                                        int qd, float sc2, float lse2, float gc, float Dc) {
  constexpr int NKK = 2 * DK / 32, NKV = 2 * DV / 32;
  f32x4 s[2], dp[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    s[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
    dp[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) mma(s[sub], load_frag(tb + (sub * (DK / 32) + ks) * 512), st.qf[ks]);
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks)
      mma(dp[sub], load_frag(tb + (NKK + sub * (DV / 32) + ks) * 512), st.dof[ks]);
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
    // dS as a bf16 hi + lo pair: a row of dS sums to zero, so dq = dS K
    // cancels and a single bf16 rounding of dS would show in it
    Frag8<T> dsf = to_frag<T>(ds), dslo;
    if constexpr (sizeof(T) == 2) split_bf16(ds, dsf, dslo);
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      const Frag8<T> kf = load_frag(tb + (NKK + NKV + dt) * 512);
      mma(st.dq[dt], kf, dsf);
      if constexpr (sizeof(T) == 2) mma(st.dq[dt], kf, dslo);
    }
  }
}

// ROWSUM = true: per row and branch, dg_c = sum_k P_k (dO . v_k) = <dO, O_c>,
// written as D_c = g_c dg_c and dz_c = dg_c g_c (1 - g_c).  ROWSUM = false: dq
// of the branches in BR (1 compressed, 2 selected, 4 window), added to dq when
// ACC.
template <typename T, int DK, int DV, bool ROWSUM, int BR = 7, bool ACC = false>
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
  float lse2[3], gc[3], Dc[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const float l = cv ? a.lse[c * BTH + row] : 0.f;
    lse2[c] = l == kNegInf ? 0.f : l * kLog2e;
    gc[c] = cv ? a.w.gates[row * 3 + c] : 0.f;
    Dc[c] = (cv && !ROWSUM) ? a.w.Dc[c * BTH + row] : 0.f;
  }
  float rsum[3] = {0.f, 0.f, 0.f};
  const int TI = 2 * DK / 32 + 2 * DV / 32 + DK / 16;
  // compressed branch
  if (BR & 1) {
    const int nv = ncmp_visible(t, dm.l, dm.d);
    const T* fb = (const T*)a.w.fckv + (size_t)(b * dm.Hkv + g) * ((dm.ncmp + 31) / 32) * TI * 512 + lane * 8;
    for (int kt = 0; kt < nv; kt += 32)
      dq_tile<T, DK, DV, ROWSUM>(st, fb + (size_t)(kt / 32) * TI * 512, kt, 0, nv, c16, qd, sc2, lse2[0], gc[0],
                                 Dc[0]);
    rsum[0] = st.rs;
    st.rs = 0.f;
  }
  const T* fb = (const T*)a.w.fkv + (size_t)(b * dm.Hkv + g) * ((dm.T + 31) / 32) * TI * 512 + lane * 8;
  // selected branch
  if (BR & 2) {
    const int* ids = a.idx + ((size_t)(b * dm.T + t) * dm.Hkv + g) * dm.n;
    const int myid = lane < dm.n ? ids[lane] : -1;
    const int nrow = wave_sel_row_len(myid, lane, dm.n, t, dm.ls);
    for (int si = 0; si < nrow; ++si) {
      const int j = __builtin_amdgcn_readlane(myid, si);
      const int lo = j * dm.ls, kend = min((j + 1) * dm.ls, t + 1);
      for (int kt = lo & ~31; kt < kend; kt += 32)
        dq_tile<T, DK, DV, ROWSUM>(st, fb + (size_t)(kt / 32) * TI * 512, kt, lo, kend, c16, qd, sc2, lse2[1],
                                   gc[1], Dc[1]);
    }
    rsum[1] = st.rs;
    st.rs = 0.f;
  }
  // window branch
  if (BR & 4) {
    const T* fw = (const T*)a.fkv_win + (size_t)(b * dm.Hkv + g) * ((dm.T + 31) / 32) * TI * 512 + lane * 8;
    const int lo = max(0, t - dm.w + 1);
    for (int kt = lo & ~31; kt <= t; kt += 32)
      dq_tile<T, DK, DV, ROWSUM>(st, fw + (size_t)(kt / 32) * TI * 512, kt, lo, t + 1, c16, qd, sc2, lse2[2],
                                 gc[2], Dc[2]);
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
    for (int dt = 0; dt < DK / 16; ++dt) {
      float v[4] = {dm.scale * st.dq[dt][0], dm.scale * st.dq[dt][1], dm.scale * st.dq[dt][2],
                    dm.scale * st.dq[dt][3]};
      if (ACC) {
        float o[4];
        load4(out + dt * 16, o);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += o[r];
      }
      store4(out + dt * 16, v[0], v[1], v[2], v[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// dq of the selected branch, added to dq: one wave per (b, t, g) as above, but
// the (block, 32-key tile) sequence of the position runs through a ring of
// DEPTH register tiles, so several tiles' gathers are in flight while one is
// computed (the branch is bound by how many bytes are outstanding).
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV>
constexpr int dqs_depth() {
  return (2 * DK / 32 + 2 * DV / 32 + DK / 16) * (sizeof(T) == 2 ? 4 : 8) * 3 <= 300 ? 3 : 2;
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256, 1) void k_bwd_dq_slc(Dims dm, BwdArgs a) {
  constexpr int NKK = 2 * DK / 32, NKV = 2 * DV / 32, TI = NKK + NKV + DK / 16;
  constexpr int DEPTH = dqs_depth<T, DK, DV>();
  struct Tile { Frag8<T> f[TI]; };
  struct Cur { int si, kt, lo, kend; };
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
  Frag8<T> qf[DK / 32], dof[DV / 32];
  f32x4 dq[DK / 16];
  {
    const T* qp = (const T*)a.q + row * DK + qd * 8;
    const T* dp = (const T*)a.d_o + row * DV + qd * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qf[ks] = cv ? load_frag(qp + ks * 32) : zero_frag<T>();
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks) dof[ks] = cv ? load_frag(dp + ks * 32) : zero_frag<T>();
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) dq[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sc2 = dm.scale * kLog2e;
  const float lraw = cv ? a.lse[BTH + row] : 0.f;
  const float lse2 = lraw == kNegInf ? 0.f : lraw * kLog2e;
  const float gc = cv ? a.w.gates[row * 3 + 1] : 0.f;
  const float Dc = cv ? a.w.Dc[BTH + row] : 0.f;
  const int* ids = a.idx + ((size_t)(b * dm.T + t) * dm.Hkv + g) * dm.n;
  const int myid = lane < dm.n ? ids[lane] : -1;
  const int nrow = wave_sel_row_len(myid, lane, dm.n, t, dm.ls);
  const T* fb = (const T*)a.w.fkv + (size_t)(b * dm.Hkv + g) * ((dm.T + 31) / 32) * TI * 512 + lane * 8;
  auto open_block = [&](Cur& c) {
    for (; c.si < nrow; ++c.si) {
      const int j = __builtin_amdgcn_readlane(myid, c.si);
      c.lo = j * dm.ls;
      c.kt = c.lo & ~31;
      c.kend = min((j + 1) * dm.ls, t + 1);
      if (c.lo < c.kend) return;
    }
    c.si = dm.n;
  };
  auto advance = [&](Cur& c) {
    c.kt += 32;
    if (c.kt < c.kend) return;
    ++c.si;
    open_block(c);
  };
  auto load_tile = [&](Tile& tl, const Cur& c) {
    const T* base = fb + (size_t)(c.kt / 32) * TI * 512;
#pragma unroll
    for (int i = 0; i < TI; ++i) tl.f[i] = load_frag(base + i * 512);
  };
  auto compute_tile = [&](const Tile& tl, const Cur& c) {
    f32x4 sv[2], dp[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      sv[sub] = dp[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) mma(sv[sub], tl.f[sub * (DK / 32) + ks], qf[ks]);
#pragma unroll
      for (int ks = 0; ks < DV / 32; ++ks) mma(dp[sub], tl.f[NKK + sub * (DV / 32) + ks], dof[ks]);
    }
    float ds[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = c.kt + qd * 8 + e;
      const bool v = key >= c.lo && key < c.kend;
      const float p = v ? fast_exp2(sv[e >> 2][e & 3] * sc2 - lse2) : 0.f;
      ds[e] = p * (gc * dp[e >> 2][e & 3] - Dc);
    }
    // dS as a bf16 hi + lo pair (dq = dS K cancels; see dq_tile)
    Frag8<T> dsf = to_frag<T>(ds), dslo;
    if constexpr (sizeof(T) == 2) split_bf16(ds, dsf, dslo);
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      mma(dq[dt], tl.f[NKK + NKV + dt], dsf);
      if constexpr (sizeof(T) == 2) mma(dq[dt], tl.f[NKK + NKV + dt], dslo);
    }
  };
  Tile ring[DEPTH];
  Cur rc[DEPTH];
  Cur lc{0, 0, 0, 0};
  open_block(lc);
#pragma unroll
  for (int r = 0; r < DEPTH; ++r) {
    rc[r] = lc;
    if (lc.si < dm.n) {
      load_tile(ring[r], lc);
      advance(lc);
    }
  }
  bool more = rc[0].si < dm.n;
  while (more) {
#pragma unroll
    for (int r = 0; r < DEPTH; ++r) {
      if (more) {
        __builtin_amdgcn_sched_barrier(0);
        compute_tile(ring[r], rc[r]);
        __builtin_amdgcn_sched_barrier(0);
        rc[r] = lc;
        if (lc.si < dm.n) {
          load_tile(ring[r], lc);
          advance(lc);
        }
        more = rc[(r + 1) % DEPTH].si < dm.n;
      }
    }
  }
  if (cv) {
    float* out = a.dq + row * DK + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      float o[4];
      load4(out + dt * 16, o);
      store4(out + dt * 16, o[0] + dm.scale * dq[dt][0], o[1] + dm.scale * dq[dt][1], o[2] + dm.scale * dq[dt][2],
             o[3] + dm.scale * dq[dt][3]);
    }
  }
}

// ---------------------------------------------------------------------------
// dq of the compressed and window branches, query-tile stationary: the query
// positions of a workgroup share every key tile of these two branches, so
// 64-key stages of the fragment-ordered tiles (key-row K, key-row V and K^T
// fragments) are copied once into LDS, double-buffered through registers, and
// each wave's columns (16*NCT (position, head) pairs) read their MFMA
// operands there.  Per 32 keys and column tile: S^T = K Q^T, dP^T = V dO^T,
// dS = P (g dP - D), dq^T += K^T dS^T.  BR: 1 compressed, 4 window.
// ---------------------------------------------------------------------------
template <typename T, int DK, int DV>
constexpr int dqt_stage_elems() { return 2 * (2 * DK / 32 + 2 * DV / 32 + DK / 16) * 512; }

template <typename T, int DK, int DV, int NCT, int NW, int BR>
__global__ __launch_bounds__(NW * 64, 2) void k_dq_tiled(Dims dm, BwdArgs a) {
  constexpr int NKK = 2 * DK / 32, NKV = 2 * DV / 32, TI = NKK + NKV + DK / 16;
  constexpr int STAGE = dqt_stage_elems<T, DK, DV>();
  constexpr int NT = NW * 64;
  constexpr int CH = STAGE / 8 / NT;            // fragments of 8 elements per thread and stage
  static_assert(CH * 8 * NT == STAGE, "stage must split evenly over the workgroup");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* stg = (T*)smem_raw;                        // [2][STAGE]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  const int G = dm.G, PW = 16 * NCT / G, PWG = NW * PW;
  const int ntiles = (dm.T + PWG - 1) / PWG;
  int unit, tile;
  xcd_map(blockIdx.x, dm.B * dm.Hkv, ntiles, unit, tile);
  const int b = unit / dm.Hkv, g = unit % dm.Hkv;
  const int twg = tile * PWG, tlast = min(dm.T - 1, twg + PWG - 1);
  const int t0 = twg + wave * PW;
  const size_t BTH = (size_t)dm.B * dm.T * dm.Hq;
  Frag8<T> qf[NCT][DK / 32], dof[NCT][DV / 32];
  int pos[NCT];
  size_t row[NCT];
  bool cvalid[NCT];
  float lse2[NCT][2], gc[NCT][2], Dc[NCT][2];
  f32x4 dq[NCT][DK / 16];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = ct * 16 + c16;
    pos[ct] = t0 + col / G;
    cvalid[ct] = pos[ct] < dm.T;
    const int hq = g * G + col % G;
    row[ct] = (size_t)(b * dm.T + min(pos[ct], dm.T - 1)) * dm.Hq + hq;
    const T* qp = (const T*)a.q + row[ct] * DK + qd * 8;
    const T* dp = (const T*)a.d_o + row[ct] * DV + qd * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qf[ct][ks] = cvalid[ct] ? load_frag(qp + ks * 32) : zero_frag<T>();
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks) dof[ct][ks] = cvalid[ct] ? load_frag(dp + ks * 32) : zero_frag<T>();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = k == 0 ? 0 : 2;
      const float l = cvalid[ct] ? a.lse[c * BTH + row[ct]] : kNegInf;
      lse2[ct][k] = l == kNegInf ? 0.f : l * kLog2e;
      gc[ct][k] = cvalid[ct] ? a.w.gates[row[ct] * 3 + c] : 0.f;
      Dc[ct][k] = cvalid[ct] ? a.w.Dc[c * BTH + row[ct]] : 0.f;
    }
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) dq[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sc2 = dm.scale * kLog2e;

  // One key stream: keys [klo, khi) of the workgroup, fragment tiles `base`
  // (nt tiles of this (b, g)); column ct sees keys [lo[ct], hi[ct]).
  auto stream = [&](const T* base, int nt, int klo, int khi, const int (&lo)[NCT], const int (&hi)[NCT], int k) {
    if (klo >= khi) return;
    const int s_first = klo & ~63;
    const int nst = (khi - s_first + 63) / 64;
    Frag8<T> pre[CH];
    auto gload = [&](int st) {
      const int tile0 = (s_first + st * 64) / 32;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int e = (tid + c * NT) * 8;            // element offset in the stage
        const int tl = tile0 + e / (TI * 512);
        pre[c] = tl < nt ? load_frag(base + (size_t)tile0 * TI * 512 + e) : zero_frag<T>();
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
        *reinterpret_cast<Frag8<T>*>(stg + (size_t)buf * STAGE + (tid + c * NT) * 8) = pre[c];
    };
    gload(0);
    __syncthreads();   // the previous stream's last stage is no longer read
    lstore(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
      if (st + 1 < nst) gload(st + 1);
      const T* sb = stg + (size_t)(st & 1) * STAGE + lane * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kt = s_first + st * 64 + h * 32;
        if (kt >= khi) break;
        const T* tb = sb + (size_t)h * TI * 512;
        f32x4 sacc[NCT][2], dpa[NCT][2];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) sacc[ct][sub] = dpa[ct][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
          for (int ks = 0; ks < DK / 32; ++ks) {
            const Frag8<T> kf = *reinterpret_cast<const Frag8<T>*>(tb + (sub * (DK / 32) + ks) * 512);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) mma(sacc[ct][sub], kf, qf[ct][ks]);
          }
#pragma unroll
          for (int ks = 0; ks < DV / 32; ++ks) {
            const Frag8<T> vf = *reinterpret_cast<const Frag8<T>*>(tb + (NKK + sub * (DV / 32) + ks) * 512);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) mma(dpa[ct][sub], vf, dof[ct][ks]);
          }
        }
        // dS as a bf16 hi + lo pair (dq = dS K cancels; see dq_tile)
        Frag8<T> dsf[NCT], dslo[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float ds[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = kt + qd * 8 + e;
            const bool v = key >= lo[ct] && key < hi[ct];
            const float pe = v ? fast_exp2(sacc[ct][e >> 2][e & 3] * sc2 - lse2[ct][k]) : 0.f;
            ds[e] = pe * (gc[ct][k] * dpa[ct][e >> 2][e & 3] - Dc[ct][k]);
          }
          dsf[ct] = to_frag<T>(ds);
          if constexpr (sizeof(T) == 2) split_bf16(ds, dsf[ct], dslo[ct]);
        }
#pragma unroll
        for (int dt = 0; dt < DK / 16; ++dt) {
          const Frag8<T> kt_f = *reinterpret_cast<const Frag8<T>*>(tb + (NKK + NKV + dt) * 512);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            mma(dq[ct][dt], kt_f, dsf[ct]);
            if constexpr (sizeof(T) == 2) mma(dq[ct][dt], kt_f, dslo[ct]);
          }
        }
      }
      if (st + 1 < nst) {
        lstore((st + 1) & 1);
      }
      __syncthreads();
    }
  };

  const int BG = b * dm.Hkv + g;
  if (BR & 1) {
    int lo[NCT], hi[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      lo[ct] = 0;
      hi[ct] = cvalid[ct] ? ncmp_visible(pos[ct], dm.l, dm.d) : 0;
    }
    const int nt = (dm.ncmp + 31) / 32;
    stream((const T*)a.w.fckv + (size_t)BG * nt * TI * 512, nt, 0, ncmp_visible(tlast, dm.l, dm.d), lo, hi, 0);
  }
  if (BR & 4) {
    int lo[NCT], hi[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      lo[ct] = max(0, pos[ct] - dm.w + 1);
      hi[ct] = cvalid[ct] ? pos[ct] + 1 : 0;
    }
    const int nt = (dm.T + 31) / 32;
    stream((const T*)a.fkv_win + (size_t)BG * nt * TI * 512, nt, max(0, twg - dm.w + 1), tlast + 1, lo, hi, 1);
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    if (!cvalid[ct]) continue;
    float* out = a.dq + row[ct] * DK + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
      store4(out + dt * 16, dm.scale * dq[ct][dt][0], dm.scale * dq[ct][dt][1], dm.scale * dq[ct][dt][2],
             dm.scale * dq[ct][dt][3]);
  }
}

// Whether the query-tile dq kernel fits (its two stages in LDS).
template <typename T, int DK, int DV>
constexpr bool dq_tiled_fits() { return 2 * dqt_stage_elems<T, DK, DV>() * sizeof(T) <= 160 * 1024; }

template <typename T, int DK, int DV, int BR>
static hipError_t launch_dq_tiled(const Dims& dm, const BwdArgs& a, hipStream_t s) {
  if constexpr (!dq_tiled_fits<T, DK, DV>()) {
    return hipErrorInvalidValue;
  } else {
    constexpr int NCT = DK >= 192 ? 1 : 2, NW = 8;   // 192-wide rows: one column tile fits the registers
    const size_t lds = 2 * (size_t)dqt_stage_elems<T, DK, DV>() * sizeof(T);
    auto kfn = k_dq_tiled<T, DK, DV, NCT, NW, BR>;
    if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    const int PWG = NW * 16 * NCT / dm.G;
    const int ntiles = (dm.T + PWG - 1) / PWG;
    kfn<<<ntiles * dm.B * dm.Hkv, NW * 64, lds, s>>>(dm, a);
    return hipGetLastError();
  }
}

// Row terms from the forward's saved fp32 branch outputs: dg_c = <dO, O_c>,
// D_c = g_c dg_c, dz_c = dg_c g_c (1 - g_c).  Memory-bound: DV/4 lanes per
// row, each reading 4 features of dO and of the three O_c.
template <typename T, int DV>
__global__ __launch_bounds__(256) void k_rowterms(Dims dm, BwdArgs a) {
  constexpr int LPR = DV / 4, RPW = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t BTH = (size_t)dm.B * dm.T * dm.Hq;
  const size_t row = ((size_t)blockIdx.x * 4 + wave) * RPW + lane / LPR;
  const int f = (lane % LPR) * 4;
  const bool live = row < BTH;
  const size_t rr = live ? row : 0;
  float d[4];
  load4((const T*)a.d_o + rr * DV + f, d);
  float v[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    float o[4];
    load4(a.ob + (c * BTH + rr) * DV + f, o);
    v[c] = d[0] * o[0] + d[1] * o[1] + d[2] * o[2] + d[3] * o[3];
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) v[c] += __shfl_xor(v[c], off);
  }
  if (!live || lane % LPR != 0) return;
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const float gc = a.w.gates[row * 3 + c];
    a.w.Dc[c * BTH + row] = gc * v[c];
    a.w.dz[row * 3 + c] = v[c] * gc * (1.f - gc);
  }
}

// ---------------------------------------------------------------------------
// dK / dV: one wave per 16 keys.
// ---------------------------------------------------------------------------
enum KvMode { KV_CMP = 0, KV_WIN = 1, KV_SLC = 2 };

// Task of one workgroup: 64 keys [k0, k0+64) (klim bounds valid keys), query
// positions p0..p1-1 (cmp, win) or plist[0..npos) (slc), partial output row
// base (cmp, slc).  Returns false when the task has no positions.
template <int MODE>
__device__ __forceinline__ bool kv_task(const Dims& dm, const BwdArgs& a, int& bg, int& k0, int& klim, int& p0,
                                        int& npos, const int*& plist, float*& outp, int W) {
  const BwdPlan& pl = a.pl;
  plist = nullptr;
  outp = nullptr;
  // Selected blocks: consecutive workgroups go to different XCDs, so the
  // (b, g) index runs fastest and every XCD receives an even share.
  const int BG = dm.B * dm.Hkv;
  if (MODE == KV_CMP) {
    // tasks in order of their first query position on each XCD (64*d keys'
    // worth of positions per group step, kSegCmp per segment)
    int kg, seg;
    span_task_order(blockIdx.x, BG, pl.nkg_cmp, pl.nseg_cmp, 64 * dm.d, kSegCmp, bg, kg, seg);
    k0 = kg * 64;
    klim = dm.ncmp;
    p0 = k0 * dm.d + dm.l - 1 + seg * kSegCmp;
    npos = max(0, min(dm.T, p0 + kSegCmp) - p0);
    outp = a.w.part_cmp + (((size_t)bg * pl.nkg_cmp + kg) * pl.nseg_cmp + seg) * 64 * W;
  } else if (MODE == KV_WIN) {
    // each XCD walks contiguous key groups of its (b, g): the groups running
    // together on it read nearly the same query rows, which its L2 then holds
    const int nkg = (dm.T + 63) / 64;
    int kg;
    xcd_map(blockIdx.x, BG, nkg, bg, kg);
    // xcd_map hands out the last groups first; with a window over the whole
    // sequence (the dense baseline) the first key groups carry the most query
    // positions, so they go first instead
    if (dm.w >= dm.T) kg = nkg - 1 - kg;
    k0 = kg * 64;
    klim = dm.T;
    p0 = k0;
    npos = min(dm.T, k0 + 63 + dm.w) - p0;
  } else {
    // segment slots of all (b, g) interleaved; unused slots hold -1
    const int kc = blockIdx.x % pl.nkc_slc;
    const int r = blockIdx.x / pl.nkc_slc;
    bg = r % BG;
    const int slot_i = r / BG;
    const int tk = a.w.task[(size_t)bg * pl.max_slc_seg + slot_i];
    if (tk < 0) return false;
    const int j = tk / pl.nseg_slc, seg = tk % pl.nseg_slc;
    const int cnt = a.w.cnt[(size_t)bg * dm.nsel + j];
    npos = min(kSegSlc, cnt - seg * kSegSlc);
    plist = a.w.list + (size_t)bg * dm.T * dm.n + a.w.lstart[(size_t)bg * dm.nsel + j] + seg * kSegSlc;
    k0 = j * dm.ls + kc * 64;
    klim = min(dm.T, (j + 1) * dm.ls);
    p0 = 0;
    const int slot = a.w.segoff[(size_t)bg * dm.nsel + j] + seg;
    outp = a.w.part_slc + ((size_t)bg * pl.max_slc_seg + slot) * dm.ls * W + (size_t)kc * 64 * W;
  }
  return npos > 0;
}

// dK / dV: one workgroup of four waves per 64 keys (16 keys per wave).  For
// every pair of query positions the workgroup stages the 2 x 16 query rows of
// q and dO in LDS, both row-major (A operand of S = Q K^T and dP = dO V^T) and
// transposed (A operand of dK^T += Q^T dS and dV^T += dO^T P), plus the rows'
// log-sum-exp, D_c and gate.  Staging is double-buffered: the next pair's
// rows are loaded into registers while the current pair is computed.  The
// positions of a selected-block list segment are read into LDS up front.
template <typename T, int DK, int DV>
struct KvStage {
  // Row strides: RS keeps 16-byte rows; TS (a multiple of 4) keeps the
  // transposed 4-row groups 8-byte aligned and spreads them over the banks.
  static constexpr int QS = DK + 8, DS = DV + 8, TS = 32 + 4;
  // A staging task is 4 consecutive rows x 8 features of q or dO.
  static constexpr int NTASK = DK + DV, NCH = (NTASK + 255) / 256;
  static constexpr size_t elems = (size_t)32 * QS + (size_t)DK * TS + (size_t)32 * DS + (size_t)DV * TS;
  static constexpr size_t bytes = elems * sizeof(T) + 3 * 32 * sizeof(float);
  Frag8<T> r[NCH][4];
  float l2, Dv, gv;
};


// Staging task u -> tensor (q or dO), feature chunk c8 and row quad rq.  Lanes
// vary the low two bits of c8 fastest (64 contiguous bytes of a row per lane
// quad), then rq, so the transposed 8-byte stores of a wave hit distinct banks.
struct KvTaskMap {
  bool is_q;
  int c8, rq;
};
template <int DK, int DV>
__device__ __forceinline__ KvTaskMap kv_task_map(int u) {
  KvTaskMap m;
  m.is_q = u < DK;
  const int v = m.is_q ? u : u - DK;
  m.c8 = (v & 3) + 4 * (v >> 5);
  m.rq = (v >> 2) & 7;
  return m;
}

template <typename T, int DK, int DV, int MODE>
__global__ __launch_bounds__(256) void k_bwd_kv(Dims dm, BwdArgs a) {
  using St = KvStage<T, DK, DV>;
  constexpr int QS = St::QS, DS = St::DS, TS = St::TS;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  int* lpos = (int*)(smem_raw + 2 * St::bytes);        // [kSegSlc] list positions (slc)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  const int W = DK + DV;
  int bg, k0, klim, p0, npos;
  const int* plist;
  float* outp;
  if (!kv_task<MODE>(dm, a, bg, k0, klim, p0, npos, plist, outp, W)) return;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int G = dm.G;
  const int c = MODE == KV_CMP ? 0 : (MODE == KV_SLC ? 1 : 2);
  const size_t BTH = (size_t)dm.B * dm.T * dm.Hq;
  if (MODE == KV_SLC) {
    for (int i = tid; i < npos; i += 256) lpos[i] = plist[i];
    __syncthreads();
  }
  auto position = [&](int ii) { return ii < npos ? (MODE == KV_SLC ? lpos[ii] : p0 + ii) : -1; };
  const int key = k0 + wave * 16 + c16;
  const bool wave_live = k0 + wave * 16 < klim;
  const bool kvalid = key < klim;
  const int kcl = min(key, klim - 1);
  const T *kr, *vr;
  if (MODE == KV_CMP) {
    kr = (const T*)a.kc + ((size_t)(b * dm.ncmp + kcl) * dm.Hkv + g) * DK;
    vr = (const T*)a.vc + ((size_t)(b * dm.ncmp + kcl) * dm.Hkv + g) * DV;
  } else {
    kr = (const T*)(MODE == KV_WIN ? a.kw : a.ks) + ((size_t)(b * dm.T + kcl) * dm.Hkv + g) * DK;
    vr = (const T*)(MODE == KV_WIN ? a.vw : a.vs) + ((size_t)(b * dm.T + kcl) * dm.Hkv + g) * DV;
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

  // Two register stages when they fit the register budget (one staging chunk
  // per thread, DK + DV <= 256): the rows of a position pair are requested two
  // pairs ahead of their compute and one pair ahead of their copy into LDS.
  // Otherwise one pair ahead, copied into LDS at the end of the same step
  // (the two stages are then never live together).
  constexpr bool kTwo = St::NCH == 1;
  St rg[2];
  // global -> registers for the position pair (pp0, pp1): rows r = i*16 + h
  auto gload = [&](auto S, int pp0, int pp1) {
    St& reg = rg[decltype(S)::value];
#pragma unroll
    for (int cc = 0; cc < St::NCH; ++cc) {
      const int u = tid + 256 * cc;
      const KvTaskMap m = kv_task_map<DK, DV>(u);
      const int pp = (m.rq >> 2) ? pp1 : pp0;
      const int h0 = (m.rq & 3) * 4;
      const int D = m.is_q ? DK : DV;
      const T* src = (const T*)(m.is_q ? a.q : a.d_o);
      const bool ok = u < St::NTASK && pp >= 0;
      // loads from a clamped row (position 0, the group's last head, feature
      // chunk 0 for threads without a task) that is always in the tensor, then
      // a select: no branch per row
      const size_t rb = ((size_t)(b * dm.T + (ok ? pp : 0)) * dm.Hq + g * G) * D + (ok ? m.c8 * 8 : 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool hv = ok && h0 + k < G;
        const Frag8<T> f = load_frag(src + rb + (size_t)min(h0 + k, G - 1) * D);
        reg.r[cc][k] = hv ? f : zero_frag<T>();
      }
    }
    if (tid < 32) {
      const int h = tid & 15, pp = (tid >> 4) ? pp1 : pp0;
      reg.l2 = 0.f; reg.Dv = 0.f; reg.gv = 0.f;
      if (pp >= 0 && h < G) {
        const size_t rr = (size_t)(b * dm.T + pp) * dm.Hq + g * G + h;
        const float l = a.lse[c * BTH + rr];
        reg.l2 = l == kNegInf ? 0.f : l * kLog2e;
        reg.Dv = a.w.Dc[c * BTH + rr];
        reg.gv = a.w.gates[rr * 3 + c];
      }
    }
  };
  // registers -> LDS buffer: row-major and transposed copies
  auto lstore = [&](auto S, int buf) {
    const St& reg = rg[decltype(S)::value];
    T* Qr = (T*)(smem_raw + (size_t)buf * St::bytes);
    T* Qt = Qr + 32 * QS;
    T* Dr = Qt + DK * TS;
    T* Dt = Dr + 32 * DS;
    float* sst = (float*)(Dt + DV * TS);
#pragma unroll
    for (int cc = 0; cc < St::NCH; ++cc) {
      const int u = tid + 256 * cc;
      if (u >= St::NTASK) break;
      const KvTaskMap m = kv_task_map<DK, DV>(u);
      T* R = m.is_q ? Qr : Dr;
      T* Tt = m.is_q ? Qt : Dt;
      const int RS = m.is_q ? QS : DS;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<Frag8<T>*>(R + (4 * m.rq + k) * RS + m.c8 * 8) = reg.r[cc][k];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        store_col4(Tt + (m.c8 * 8 + e) * TS + 4 * m.rq, frag_at(reg.r[cc][0], e), frag_at(reg.r[cc][1], e),
                   frag_at(reg.r[cc][2], e), frag_at(reg.r[cc][3], e));
    }
    if (tid < 32) {
      sst[tid] = reg.l2;
      sst[32 + tid] = reg.Dv;
      sst[64 + tid] = reg.gv;
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  gload(S0{}, position(0), position(1));
  if (kTwo && 2 < npos) gload(S1{}, position(2), position(3));
  lstore(S0{}, 0);
  __syncthreads();
  // Pair pi/2 is computed from LDS buffer buf = (pi/2) & 1.  With two stages
  // its registers were stage buf (a compile-time index: that loop is unrolled
  // by two pairs); with one stage everything goes through stage 0.
  auto step = [&](auto RS, int buf, int pi) {
    constexpr int rs = decltype(RS)::value;
    int pos[2] = {position(pi), position(pi + 1)};
    if constexpr (kTwo) {
      if (pi + 4 < npos) gload(RS, position(pi + 4), position(pi + 5));
    } else {
      if (pi + 2 < npos) gload(S0{}, position(pi + 2), position(pi + 3));
    }
    const T* Qr = (const T*)(smem_raw + (size_t)buf * St::bytes);
    const T* Qt = Qr + 32 * QS;
    const T* Dr = Qt + DK * TS;
    const T* Dt = Dr + 32 * DS;
    const float* slse = (const float*)(Dt + DV * TS);
    const float* sD = slse + 32;
    const float* sg = sD + 32;
    if (wave_live) {
      float pg[2][4], dsv[2][4];
      // S and dP of both 16-row tiles first: four independent MFMA chains
      f32x4 sacc[2], dpacc[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        sacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        dpacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          mma(sacc[i], *reinterpret_cast<const Frag8<T>*>(Qr + (i * 16 + c16) * QS + ks * 32 + qd * 8), kf[ks]);
#pragma unroll
      for (int ks = 0; ks < DV / 32; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          mma(dpacc[i], *reinterpret_cast<const Frag8<T>*>(Dr + (i * 16 + c16) * DS + ks * 32 + qd * 8), vf[ks]);
      // Row terms without branches: a lane's four rows are consecutive in the
      // staged log-sum-exp, D_c and gate arrays.  Staged rows past the
      // positions or heads hold 0 there and zero q / dO, so every lane
      // evaluates finite values and the mask only selects them.
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = pos[i];
        bool pv = t >= 0 && kvalid;
        if (MODE == KV_CMP) pv = pv && key < ncmp_visible(t, dm.l, dm.d);
        else if (MODE == KV_WIN) pv = pv && key <= t && t <= key + dm.w - 1;
        else pv = pv && key <= t;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(slse + i * 16 + qd * 4);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(sD + i * 16 + qd * 4);
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(sg + i * 16 + qd * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool v = pv && (qd * 4 + r) < G;
          const float p = fast_exp2(sacc[i][r] * sc2 - l4[r]);
          pg[i][r] = v ? p * g4[r] : 0.f;
          dsv[i][r] = v ? p * (g4[r] * dpacc[i][r] - d4[r]) : 0.f;
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
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) {
        const T* src = Dt + (dt * 16 + c16) * TS + qd * 4;
        float x[8];
        load4(src, x);
        load4(src + 16, x + 4);
        const Frag8<T> xf = to_frag<T>(x);
        mma(dv[dt], xf, pfr);
        if constexpr (sizeof(T) == 2) mma(dv[dt], xf, plo);
      }
#pragma unroll
      for (int dt = 0; dt < DK / 16; ++dt) {
        const T* src = Qt + (dt * 16 + c16) * TS + qd * 4;
        float x[8];
        load4(src, x);
        load4(src + 16, x + 4);
        const Frag8<T> xf = to_frag<T>(x);
        mma(dk[dt], xf, dsf);
        if constexpr (sizeof(T) == 2) mma(dk[dt], xf, dslo);
      }
    }
    if (pi + 2 < npos) {
      if constexpr (kTwo) lstore(std::integral_constant<int, rs ^ 1>{}, buf ^ 1);
      else lstore(S0{}, buf ^ 1);
    }
    __syncthreads();
  };
  if constexpr (kTwo) {
    for (int pi = 0; pi < npos; pi += 4) {
      step(S0{}, 0, pi);
      if (pi + 2 < npos) step(S1{}, 1, pi + 2);
    }
  } else {
    for (int pi = 0; pi < npos; pi += 2) step(S0{}, (pi >> 1) & 1, pi);
  }
  if (!wave_live) return;
  // write: lane holds key column c16, features dt*16 + 4qd + r
  if (MODE == KV_WIN) {
    if (!kvalid) return;
    float* dkp = a.dkw + ((size_t)(b * dm.T + key) * dm.Hkv + g) * DK + qd * 4;
    float* dvp = a.dvw + ((size_t)(b * dm.T + key) * dm.Hkv + g) * DV + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
      store4(dkp + dt * 16, dm.scale * dk[dt][0], dm.scale * dk[dt][1], dm.scale * dk[dt][2], dm.scale * dk[dt][3]);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) store4(dvp + dt * 16, dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]);
  } else {
    float* op = outp + (size_t)(wave * 16 + c16) * W + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
      store4(op + dt * 16, dm.scale * dk[dt][0], dm.scale * dk[dt][1], dm.scale * dk[dt][2], dm.scale * dk[dt][3]);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) store4(op + DK + dt * 16, dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]);
  }
}

template <typename T, int DK, int DV>
static size_t kv_lds() {
  return 2 * KvStage<T, DK, DV>::bytes + kSegSlc * sizeof(int);
}

// Segment sums of the dK/dV partials, in segment order (deterministic).  A
// thread owns kRedVec vectors of 4 consecutive features of one key; grid.y
// splits a 64-key group's (dk+dv)/4-vector rows over workgroups, so every
// thread's loads are independent and can be in flight together.
constexpr int kRedVec = 4;

// compressed keys: dkc/dvc [B,Hkv,ncmp,D] = sum over the query segments
__global__ __launch_bounds__(256) void k_reduce_cmp(Dims dm, BwdArgs a) {
  const BwdPlan& pl = a.pl;
  const int W4 = (dm.dk + dm.dv) / 4;
  const int r = blockIdx.x;              // (bg, kg)
  const int kg = r % pl.nkg_cmp, bg = r / pl.nkg_cmp;
  // segments of this key group start at its first key's first visible position
  const int pf = (kg * 64) * dm.d + dm.l - 1;
  const int nseg = pf < dm.T ? min(pl.nseg_cmp, (dm.T - pf + kSegCmp - 1) / kSegCmp) : 0;
  const f32x4* __restrict__ part = reinterpret_cast<const f32x4*>(a.w.part_cmp) + (size_t)r * pl.nseg_cmp * 64 * W4;
  const size_t sstride = (size_t)64 * W4;
  float* __restrict__ dkc = a.w.dkc;
  float* __restrict__ dvc = a.w.dvc;
#pragma unroll
  for (int q = 0; q < kRedVec; ++q) {
    const int v = (blockIdx.y * kRedVec + q) * 256 + threadIdx.x;
    const int kk = v / W4, e = (v % W4) * 4, key = kg * 64 + kk;
    if (kk >= 64 || key >= dm.ncmp) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int seg = 0; seg < nseg; ++seg) acc += part[seg * sstride + v];
    float* dst = e < dm.dk ? dkc + ((size_t)bg * dm.ncmp + key) * dm.dk + e
                           : dvc + ((size_t)bg * dm.ncmp + key) * dm.dv + (e - dm.dk);
    *reinterpret_cast<f32x4*>(dst) = acc;
  }
}

// selected blocks: dks/dvs += sum over the block's list segments
__global__ __launch_bounds__(256) void k_reduce_slc(Dims dm, BwdArgs a) {
  const BwdPlan& pl = a.pl;
  const int W4 = (dm.dk + dm.dv) / 4;
  const int j = blockIdx.x % dm.nsel, bg = blockIdx.x / dm.nsel;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int cnt = a.w.cnt[(size_t)bg * dm.nsel + j];
  if (cnt == 0) return;
  const int nseg = (cnt + kSegSlc - 1) / kSegSlc;
  const int slot0 = a.w.segoff[(size_t)bg * dm.nsel + j];
  const f32x4* __restrict__ part =
      reinterpret_cast<const f32x4*>(a.w.part_slc) + ((size_t)bg * pl.max_slc_seg + slot0) * dm.ls * W4;
  const size_t sstride = (size_t)dm.ls * W4;
  float* __restrict__ dks = a.dks;
  float* __restrict__ dvs = a.dvs;
#pragma unroll
  for (int q = 0; q < kRedVec; ++q) {
    const int v = (blockIdx.y * kRedVec + q) * 256 + threadIdx.x;
    const int kk = v / W4, e = (v % W4) * 4, key = j * dm.ls + kk;
    if (kk >= dm.ls || key >= dm.T) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sg = 0; sg < nseg; ++sg) acc += part[sg * sstride + v];
    float* dst = e < dm.dk ? dks + ((size_t)(b * dm.T + key) * dm.Hkv + g) * dm.dk + e
                           : dvs + ((size_t)(b * dm.T + key) * dm.Hkv + g) * dm.dv + (e - dm.dk);
    f32x4 d = *reinterpret_cast<const f32x4*>(dst);
    d += acc;
    *reinterpret_cast<f32x4*>(dst) = d;
  }
}

// ---------------------------------------------------------------------------
// Reverse index: positions that selected each block, ascending.
// ---------------------------------------------------------------------------
// The two per-chunk kernels below run one wave per workgroup: its LDS updates
// happen in program order, so the chunk's positions follow one another
// without a barrier, and the index rows of kRevBatch positions are requested
// together (the position clamped to the chunk, the slot to the row, so every
// load is in bounds and unconditional).
constexpr int kRevBatch = 8;

__global__ __launch_bounds__(64) void k_rev_hist(Dims dm, BwdArgs a) {
  extern __shared__ int hist[];
  const BwdPlan& pl = a.pl;
  const int ch = blockIdx.x % pl.nchunk, bg = blockIdx.x / pl.nchunk;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  for (int j = threadIdx.x; j < dm.nsel; j += 64) hist[j] = 0;
  __syncthreads();
  const int t0 = ch * kRevChunk, t1 = min(dm.T, t0 + kRevChunk);
  const int lane = threadIdx.x, slot = min(lane, dm.n - 1);
  for (int tb = t0; tb < t1; tb += kRevBatch) {
    int jv[kRevBatch];
#pragma unroll
    for (int u = 0; u < kRevBatch; ++u)
      jv[u] = a.idx[((size_t)(b * dm.T + min(tb + u, t1 - 1)) * dm.Hkv + g) * dm.n + slot];
#pragma unroll
    for (int u = 0; u < kRevBatch; ++u) {
      const int t = tb + u;
      if (t >= t1) break;
      // only the row's usable prefix counts (distinct, causal blocks)
      const int j = lane < dm.n ? jv[u] : -1;
      if (lane < wave_sel_row_len(j, lane, dm.n, t, dm.ls)) hist[j] += 1;
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < dm.nsel; j += 64)
    a.w.hist[((size_t)bg * pl.nchunk + ch) * dm.nsel + j] = hist[j];
}

// Per (b, g): each block's count, first list entry and first segment slot,
// the segment-slot -> (block, segment) table, and each chunk's offset into
// every block's list.  The counts stay in LDS; every thread takes a
// contiguous range of blocks, and an exclusive scan over the threads gives
// each range its first entry and slot, so the table is in block order as a
// serial walk would write it.  LDS: nsel + 512 ints.
__global__ __launch_bounds__(256) void k_rev_scan(Dims dm, BwdArgs a) {
  extern __shared__ int sc[];
  const BwdPlan& pl = a.pl;
  const int bg = blockIdx.x, tid = threadIdx.x;
  int* cnt_s = sc;                                   // [nsel] counts, then list starts
  int* part_c = sc + ((dm.nsel + 3) & ~3);           // [256] entries per thread range
  int* part_s = part_c + 256;                        // [256] segments per thread range
  for (int j = tid; j < dm.nsel; j += 256) {
    int tot = 0;
    for (int ch = 0; ch < pl.nchunk; ++ch) tot += a.w.hist[((size_t)bg * pl.nchunk + ch) * dm.nsel + j];
    a.w.cnt[(size_t)bg * dm.nsel + j] = tot;
    cnt_s[j] = tot;
  }
  __syncthreads();
  const int per = (dm.nsel + 255) / 256;
  const int j0 = min(tid * per, dm.nsel), j1 = min(j0 + per, dm.nsel);
  int c = 0, ns = 0;
  for (int j = j0; j < j1; ++j) {
    c += cnt_s[j];
    ns += (cnt_s[j] + kSegSlc - 1) / kSegSlc;
  }
  part_c[tid] = c;
  part_s[tid] = ns;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {   // inclusive scan over the threads
    const int vc = tid >= off ? part_c[tid - off] : 0, vs = tid >= off ? part_s[tid - off] : 0;
    __syncthreads();
    part_c[tid] += vc;
    part_s[tid] += vs;
    __syncthreads();
  }
  int run = part_c[tid] - c, srun = part_s[tid] - ns;
  const int nslots = part_s[255];
  int* task = a.w.task + (size_t)bg * pl.max_slc_seg;
  for (int j = j0; j < j1; ++j) {
    const int cj = cnt_s[j], nsj = (cj + kSegSlc - 1) / kSegSlc;
    a.w.lstart[(size_t)bg * dm.nsel + j] = run;
    a.w.segoff[(size_t)bg * dm.nsel + j] = srun;
    for (int sg = 0; sg < nsj; ++sg) task[srun + sg] = j * pl.nseg_slc + sg;
    cnt_s[j] = run;   // this thread's own block: its list start from here on
    run += cj;
    srun += nsj;
  }
  for (int i = nslots + tid; i < pl.max_slc_seg; i += 256) task[i] = -1;
  __syncthreads();
  for (int j = tid; j < dm.nsel; j += 256) {
    int r = cnt_s[j];
    for (int ch = 0; ch < pl.nchunk; ++ch) {
      const size_t o = ((size_t)bg * pl.nchunk + ch) * dm.nsel + j;
      a.w.offc[o] = r;
      r += a.w.hist[o];
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
  const int lane = threadIdx.x, slot = min(lane, dm.n - 1);
  for (int tb = t0; tb < t1; tb += kRevBatch) {
    int jv[kRevBatch];
#pragma unroll
    for (int u = 0; u < kRevBatch; ++u)
      jv[u] = a.idx[((size_t)(b * dm.T + min(tb + u, t1 - 1)) * dm.Hkv + g) * dm.n + slot];
#pragma unroll
    for (int u = 0; u < kRevBatch; ++u) {
      const int t = tb + u;
      if (t >= t1) break;
      const int j = lane < dm.n ? jv[u] : -1;
      // positions enter each block's list in increasing order
      if (lane < wave_sel_row_len(j, lane, dm.n, t, dm.ls)) list[cur[j]++] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// Strided fp32 GEMM on MFMA: C[m,n] (+)= sum_k A[m*sam + k*sak] * B[k*sbk + n*sbn].
// 64x64 output tile per workgroup, k steps of 32 staged through LDS.
// ---------------------------------------------------------------------------
// Column sums out[c] = sum_r in[r*ld + c] in two stages with a fixed order:
// row split z sums rows z, z + nsplit, ...; then the splits are added in
// order.  Each stage keeps eight running sums (rows 8 apart in its sequence,
// so that eight loads are in flight), added pairwise at the end.
__device__ __forceinline__ float sum8(const float (&acc)[8]) {
  return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

__global__ __launch_bounds__(256) void k_colsum_part(int R, int Cn, long long ld, int nsplit,
                                                     const float* __restrict__ in, float* __restrict__ part) {
  const int c = blockIdx.x * 256 + threadIdx.x, z = blockIdx.y;
  if (c >= Cn) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int r = z;
  for (; r + 7 * nsplit < R; r += 8 * nsplit) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += in[(long long)(r + u * nsplit) * ld + c];
  }
  for (; r < R; r += nsplit) acc[0] += in[(long long)r * ld + c];
  part[(size_t)z * Cn + c] = sum8(acc);
}

__global__ __launch_bounds__(256) void k_colsum_fin(int Cn, int nsplit, const float* __restrict__ part,
                                                    float* __restrict__ out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= Cn) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int z = 0;
  for (; z + 8 <= nsplit; z += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += part[(size_t)(z + u) * Cn + c];
  }
  for (; z < nsplit; ++z) acc[0] += part[(size_t)z * Cn + c];
  out[c] = sum8(acc);
}

// A reduction GEMM of the backward: with bf16 I/O the library's bf16 MFMA
// GEMM (fp32 operands as bf16 hi + lo parts, fp32 accumulation; split over
// k when `split`, at most kMaxSplit ways), when the operand layouts suit it;
// otherwise, and with fp32 I/O, the exact fp32 GEMM.
template <typename T>
static hipError_t bwd_gemm(const Gemm& g, bool a_f32, bool b_f32, bool split, float* part, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    const MmArgs m{g.M, g.N, g.K, g.A, g.sam, g.sak, g.B, g.sbk, g.sbn, g.C, g.ldc, g.accumulate, 0};
    if (mm_supported(m, a_f32, b_f32)) return mm(m, a_f32, b_f32, split ? mm_split(m, kMaxSplit) : 1, part, s);
  }
  return gemm_exact(g, a_f32, b_f32, split ? part : nullptr, s);
}

static hipError_t colsum(int R, int Cn, long long ld, const float* in, float* out, float* part, hipStream_t s) {
  const int nsplit = min(kMaxSplit, max(1, R / 64));
  dim3 g1((Cn + 255) / 256, nsplit);
  k_colsum_part<<<g1, 256, 0, s>>>(R, Cn, ld, nsplit, in, part);
  k_colsum_fin<<<(Cn + 255) / 256, 256, 0, s>>>(Cn, nsplit, part, out);
  return hipGetLastError();
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

// The MLP gradient da = dh * gelu'(act), moved to the sub-block row layout of
// the GEMM1 rows: compressed key i of head (b, g) goes to row bg*nsub + R-1 + i,
// and rows bg*nsub .. bg*nsub + R-2 (and R-1 rows past the last head) hold
// zeros.  Key i reads sub-blocks i .. i+R-1, one per W1 chunk r, so the rows
// that pair with sub-block row m under chunk r are this layout shifted by
// R-1-r rows, for every head at once.  da is kept in fp32; with bf16 I/O the
// GEMMs take it as a bf16 hi part plus the bf16 rounding of the remainder
// (~16 mantissa bits).  dh is overwritten with da (its column sum is db1).
__global__ __launch_bounds__(256) void k_phi_da(Dims dm, int nsub, const float* __restrict__ act,
                                                float* __restrict__ dh, float* __restrict__ dap) {
  const int H = dm.hidden, R = dm.l / dm.d;
  const size_t BG = (size_t)dm.B * dm.Hkv, rows_p = BG * nsub + R - 1;
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows_p * H) return;
  const size_t p = id / H;
  const int o = (int)(id % H);
  const size_t bg = p / nsub;
  const int i = (int)(p % nsub) - (R - 1);
  float v = 0.f;
  if (bg < BG && i >= 0) {
    const size_t k = (bg * dm.ncmp + i) * H + o;
    const float x = act[k];
    const float cdf = 0.5f * (1.f + erff(x * 0.70710678118654752f));
    const float pdf = 0.3989422804014327f * expf(-0.5f * x * x);
    v = dh[k] * (cdf + x * pdf);
    dh[k] = v;
  }
  dap[id] = v;
}

// Position-embedding part of dW1: every compressed key adds pe to its sub-block
// rows, so dW1[x][o] gains pe[x] * sum of da[., o] = pe[x] * db1[o].
template <typename T>
__global__ __launch_bounds__(256) void k_phi_dw1_pe(size_t n, int H, const T* __restrict__ pe,
                                                    const float* __restrict__ db1, float* __restrict__ dw1) {
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= n) return;
  dw1[id] += to_f32(pe[id / H]) * db1[id % H];
}

// dpe = sum over keys of da W1^T = db1 W1^T: one wave per pe element.
template <typename T>
__global__ __launch_bounds__(256) void k_phi_dpe(int n, int H, const T* __restrict__ w1,
                                                 const float* __restrict__ db1, float* __restrict__ dpe) {
  const int x = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (x >= n) return;
  float acc = 0.f;
  for (int o = lane; o < H; o += 64) acc += db1[o] * to_f32(w1[(size_t)x * H + o]);
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (lane == 0) dpe[x] = acc;
}

// Token gradient from phi: dx[b, tok, g, e] += dxs[bg*nsub + tok/d][(tok%d)*D + e]
// (MLP: the GEMMs already summed the blocks covering each sub-block), or the
// sum over blocks i covering tok of dcmp[(bg,i)][e] / l (mean).
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
  if (mlp) {
    const int nsub = dm.ncmp + dm.l / dm.d - 1;
    if (tok < nsub * dm.d)
      dx[id] += src[((size_t)bg * nsub + tok / dm.d) * dm.d * D + (size_t)(tok % dm.d) * D + e];
    return;
  }
  // blocks i with i*d <= tok < i*d + l, 0 <= i < ncmp
  int ilo = tok - dm.l + 1;
  ilo = ilo <= 0 ? 0 : (ilo + dm.d - 1) / dm.d;
  const int ihi = min(tok / dm.d, dm.ncmp - 1);
  float s = 0.f;
  for (int i = ilo; i <= ihi; ++i) s += src[((size_t)bg * dm.ncmp + i) * D + e] / (float)dm.l;
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
  if ((e = launch_phi_gemm1(dm, D, nsub, xsrc, w.pe, w.w1, a.w.arows, a.w.y, a.w.pe_part, s)) != hipSuccess)
    return e;
  k_phi_act<T><<<(unsigned)((rows * H + 255) / 256), 256, 0, s>>>(dm, a.w.y, (const T*)w.b1, a.w.act, a.w.hid);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // db2 = colsum(dout); dW2 = hid^T dout
  if ((e = colsum((int)rows, D, D, dcmp, (float*)gr.b2, a.w.gpart, s)) != hipSuccess) return e;
  {
    Gemm g{H, D, (int)rows, a.w.hid, 1, H, dcmp, D, 1, (float*)gr.w2, D, 0};
    if ((e = bwd_gemm<T>(g, true, true, true, a.w.gpart, s)) != hipSuccess) return e;
  }
  // dh = dout W2^T; da = dh * gelu'(act)
  {
    Gemm g{(int)rows, H, D, dcmp, D, 1, w.w2, 1, D, a.w.dh, H, 0};
    if ((e = bwd_gemm<T>(g, true, sizeof(T) == 4, false, nullptr, s)) != hipSuccess) return e;
  }
  const size_t Mmain = (size_t)dm.B * dm.Hkv * nsub, rows_p = Mmain + R - 1;
  k_phi_da<<<(unsigned)((rows_p * H + 255) / 256), 256, 0, s>>>(dm, nsub, a.w.act, a.w.dh, a.w.dap);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = colsum((int)rows, H, H, a.w.dh, (float*)gr.b1, a.w.gpart, s)) != hipSuccess) return e;
  const bool bf = sizeof(T) == 2;
  const int dD = dm.d * D;
  auto da_rows = [&](int shift) { return a.w.dap + (size_t)shift * H; };
  // dW1 chunk r = (sub-block rows)^T (da shifted by R-1-r), plus the pe part;
  // the sum runs over the sub-block rows, split for parallelism
  for (int r = 0; r < R; ++r) {
    float* dw1 = (float*)gr.w1 + (size_t)r * dD * H;
    if (bf) {
      const MmArgs g{dD, H, (int)Mmain, a.w.arows, 1, dD, da_rows(R - 1 - r), H, 1, dw1, H, 0, 0};
      e = mm(g, false, true, mm_split(g, kW1Split), a.w.gpart, s);
    } else {
      const Gemm g{dD, H, (int)Mmain, a.w.arows, 1, dD, da_rows(R - 1 - r), H, 1, dw1, H, 0};
      e = gemm_exact(g, true, true, a.w.gpart, s);
    }
    if (e != hipSuccess) return e;
  }
  {
    const size_t n = (size_t)dm.l * D * H;
    k_phi_dw1_pe<T><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(n, H, (const T*)w.pe, (const float*)gr.b1,
                                                                 (float*)gr.w1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // token gradient per sub-block: sum over chunks of (da shifted by R-1-r) W1_r^T
  for (int r = 0; r < R; ++r) {
    const void* w1r = (const char*)w.w1 + (size_t)r * dD * H * sizeof(T);
    if (bf) {
      const MmArgs g{(int)Mmain, dD, H, da_rows(R - 1 - r), H, 1, w1r, 1, H, a.w.dxs, dD, r > 0, 0};
      e = mm(g, true, false, 1, nullptr, s);
    } else {
      const Gemm g{(int)Mmain, dD, H, da_rows(R - 1 - r), H, 1, w1r, 1, H, a.w.dxs, dD, r > 0};
      e = gemm_exact(g, true, true, nullptr, s);
    }
    if (e != hipSuccess) return e;
  }
  k_phi_dpe<T><<<(unsigned)((dm.l * D + 3) / 4), 256, 0, s>>>(dm.l * D, H, (const T*)w.w1, (const float*)gr.b1,
                                                              (float*)gr.pe);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t total = (size_t)dm.B * dm.T * dm.Hkv * D;
  k_phi_dx<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(dm, D, a.w.dxs, 1, dx);
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
  if ((e = launch_gate_mlp(dm, dm.B * dm.T, a.x, a.wg, GateMlp{args->gate_mlp.w1, args->gate_mlp.b1, args->gate_mlp.b2},
                           a.w.ghid, a.w.gpre, a.w.gates, s)) != hipSuccess)
    return e;
  // stage 1: fragment tiles of (k, v, k^T) and (k_cmp, v_cmp, k_cmp^T) for the dq passes
  if ((e = mark()) != hipSuccess) return e;
  {
    const int ti = bwd_tile_ins(dm);
    const int n1 = 2 * DK / 32, n2 = n1 + 2 * DV / 32;
    if ((e = launch_frag_pack(dm, DK, dm.T, a.ks, a.w.fkv, ti, 0, false, s)) != hipSuccess ||
        (e = launch_frag_pack(dm, DV, dm.T, a.vs, a.w.fkv, ti, n1, false, s)) != hipSuccess ||
        (e = launch_frag_pack(dm, DK, dm.T, a.ks, a.w.fkv, ti, n2, true, s)) != hipSuccess)
      return e;
    if (a.split &&
        ((e = launch_frag_pack(dm, DK, dm.T, a.kw, a.w.fkvw, ti, 0, false, s)) != hipSuccess ||
         (e = launch_frag_pack(dm, DV, dm.T, a.vw, a.w.fkvw, ti, n1, false, s)) != hipSuccess ||
         (e = launch_frag_pack(dm, DK, dm.T, a.kw, a.w.fkvw, ti, n2, true, s)) != hipSuccess))
      return e;
    if (dm.ncmp > 0 &&
        ((e = launch_frag_pack(dm, DK, dm.ncmp, a.kc, a.w.fckv, ti, 0, false, s)) != hipSuccess ||
         (e = launch_frag_pack(dm, DV, dm.ncmp, a.vc, a.w.fckv, ti, n1, false, s)) != hipSuccess ||
         (e = launch_frag_pack(dm, DK, dm.ncmp, a.kc, a.w.fckv, ti, n2, true, s)) != hipSuccess))
      return e;
  }
  // stage 2: row terms D_c, dz (from the saved branch outputs when given,
  // else recomputed from the probabilities), then dq
  if ((e = mark()) != hipSuccess) return e;
  if (a.ob) {
    const size_t rows = BTH, per_block = 4 * (64 / (DV / 4));
    k_rowterms<T, DV><<<(unsigned)((rows + per_block - 1) / per_block), 256, 0, s>>>(dm, a);
  } else {
    k_bwd_dq<T, DK, DV, true><<<((dm.T + 3) / 4) * BG, 256, 0, s>>>(dm, a);
  }
  if constexpr (dq_tiled_fits<T, DK, DV>()) {
    // compressed and window branches query-tile stationary, then the selected
    // branch per position, added
    if ((e = launch_dq_tiled<T, DK, DV, 5>(dm, a, s)) != hipSuccess) return e;
    k_bwd_dq_slc<T, DK, DV><<<((dm.T + 3) / 4) * BG, 256, 0, s>>>(dm, a);
  } else {
    k_bwd_dq<T, DK, DV, false><<<((dm.T + 3) / 4) * BG, 256, 0, s>>>(dm, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // stage 3: compressed keys
  const size_t klds = kv_lds<T, DK, DV>();
  if (klds > 64 * 1024) {
    hipFuncSetAttribute((const void*)k_bwd_kv<T, DK, DV, KV_CMP>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)klds);
    hipFuncSetAttribute((const void*)k_bwd_kv<T, DK, DV, KV_WIN>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)klds);
    hipFuncSetAttribute((const void*)k_bwd_kv<T, DK, DV, KV_SLC>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)klds);
  }
  if ((e = mark()) != hipSuccess) return e;
  if (dm.ncmp > 0) {
    k_bwd_kv<T, DK, DV, KV_CMP><<<BG * pl.nkg_cmp * pl.nseg_cmp, 256, klds, s>>>(dm, a);
    {
      const int nv = 64 * ((dm.dk + dm.dv) / 4);
      k_reduce_cmp<<<dim3(BG * pl.nkg_cmp, (nv + 256 * kRedVec - 1) / (256 * kRedVec)), 256, 0, s>>>(dm, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // stage 4: window keys (writes dkw, dvw); with independent K/V per branch the
  // selected branch's and phi's gradients start from zero instead of adding to it
  if ((e = mark()) != hipSuccess) return e;
  if (a.split) {
    const size_t nk = (size_t)dm.B * dm.T * dm.Hkv * DK, nv = (size_t)dm.B * dm.T * dm.Hkv * DV;
    if ((e = zero_f32(a.dks, nk, s)) != hipSuccess || (e = zero_f32(a.dvs, nv, s)) != hipSuccess ||
        (e = zero_f32(a.dk, nk, s)) != hipSuccess || (e = zero_f32(a.dv, nv, s)) != hipSuccess)
      return e;
  }
  k_bwd_kv<T, DK, DV, KV_WIN><<<BG * ((dm.T + 63) / 64), 256, klds, s>>>(dm, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // stage 5: selected blocks (adds into dks, dvs)
  if ((e = mark()) != hipSuccess) return e;
  k_rev_hist<<<BG * pl.nchunk, 64, dm.nsel * sizeof(int), s>>>(dm, a);
  {
    const size_t lds = ((size_t)((dm.nsel + 3) & ~3) + 512) * sizeof(int);
    if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void*)k_rev_scan, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    k_rev_scan<<<BG, 256, lds, s>>>(dm, a);
  }
  k_rev_fill<<<BG * pl.nchunk, 64, dm.nsel * sizeof(int), s>>>(dm, a);
  k_bwd_kv<T, DK, DV, KV_SLC><<<BG * pl.max_slc_seg * pl.nkc_slc, 256, klds, s>>>(dm, a);
  {
    const int nv = dm.ls * ((dm.dk + dm.dv) / 4);
    k_reduce_slc<<<dim3(BG * dm.nsel, (nv + 256 * kRedVec - 1) / (256 * kRedVec)), 256, 0, s>>>(dm, a);
  }
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
  // stage 7: gate weights (and the gate input's gradient when asked for)
  if ((e = mark()) != hipSuccess) return e;
  {
    const int ntok = dm.B * dm.T, HO = 3 * dm.Hq;
    float* dx = (float*)args->dx;
    if (dm.Cg == 0) {
      // dW_g = x^T dz; dx = dz W_g^T
      Gemm g{dm.C, HO, ntok, a.x, 1, dm.C, a.w.dz, HO, 1, a.dwg, HO, 0};
      if ((e = bwd_gemm<T>(g, sizeof(T) == 4, true, true, a.w.gpart, s)) != hipSuccess) return e;
      if (dx) {
        Gemm gx{ntok, dm.C, HO, a.w.dz, HO, 1, a.wg, 1, HO, dx, dm.C, 0};
        if ((e = gemm_exact(gx, true, sizeof(T) == 4, nullptr, s)) != hipSuccess) return e;
      }
    } else {
      const nsa_gate_grads& gg = args->d_gate_mlp;
      const int Cg = dm.Cg;
      // output layer: dW2 = hid^T dz, db2 = colsum(dz), dhid = dz W2^T
      Gemm g2{Cg, HO, ntok, a.w.ghid, 1, Cg, a.w.dz, HO, 1, a.dwg, HO, 0};
      if ((e = gemm_exact(g2, true, true, a.w.gpart, s)) != hipSuccess) return e;
      if ((e = colsum(ntok, HO, HO, a.w.dz, (float*)gg.b2, a.w.gpart, s)) != hipSuccess) return e;
      Gemm gh{ntok, Cg, HO, a.w.dz, HO, 1, a.wg, 1, HO, a.w.gdh, Cg, 0};
      if ((e = gemm_exact(gh, true, sizeof(T) == 4, nullptr, s)) != hipSuccess) return e;
      // GELU: da = dhid * gelu'(pre); first layer: dW1 = x^T da, db1 = colsum(da), dx = da W1^T
      k_phi_dact<<<(unsigned)(((size_t)ntok * Cg + 255) / 256), 256, 0, s>>>((size_t)ntok * Cg, a.w.gpre, a.w.gdh);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = colsum(ntok, Cg, Cg, a.w.gdh, (float*)gg.b1, a.w.gpart, s)) != hipSuccess) return e;
      Gemm g1{dm.C, Cg, ntok, a.x, 1, dm.C, a.w.gdh, Cg, 1, (float*)gg.w1, Cg, 0};
      if ((e = gemm_exact(g1, sizeof(T) == 4, true, a.w.gpart, s)) != hipSuccess) return e;
      if (dx) {
        Gemm gx{ntok, dm.C, Cg, a.w.gdh, Cg, 1, args->gate_mlp.w1, 1, Cg, dx, dm.C, 0};
        if ((e = gemm_exact(gx, true, sizeof(T) == 4, nullptr, s)) != hipSuccess) return e;
      }
    }
  }
  return mark();
}

hipError_t launch_bwd(const Dims& dm, const nsa_bwd_args* args, void* ws, hipStream_t s, void* const* events) {
  BwdArgs a;
  a.q = args->q; a.k = args->k; a.v = args->v; a.x = args->x; a.wg = args->w_gate;
  a.kc = args->k_cmp; a.vc = args->v_cmp; a.d_o = args->d_o;
  a.lse = (const float*)args->lse; a.idx = (const int*)args->idx;
  a.ob = (const float*)args->o_branch;
  a.dq = (float*)args->dq; a.dk = (float*)args->dk; a.dv = (float*)args->dv; a.dwg = (float*)args->dw_gate;
  bwd_carve(dm, ws, &a.w);
  a.split = args->k_slc != nullptr;
  if (a.split) {
    a.ks = args->k_slc; a.vs = args->v_slc; a.kw = args->k_win; a.vw = args->v_win;
    a.dks = (float*)args->dk_slc; a.dvs = (float*)args->dv_slc;
    a.dkw = (float*)args->dk_win; a.dvw = (float*)args->dv_win;
    a.fkv_win = a.w.fkvw;
  } else {
    a.ks = a.kw = a.k; a.vs = a.vw = a.v;
    a.dks = a.dkw = a.dk; a.dvs = a.dvw = a.dv;
    a.fkv_win = a.w.fkv;
  }
  a.pl = bwd_plan(dm);
  const bool bf = dm.io == IO_BF16;
  if (dm.dk == 64 && dm.dv == 64) return bf ? bwd_impl<bf16, 64, 64>(dm, args, a, s, events) : bwd_impl<float, 64, 64>(dm, args, a, s, events);
  if (dm.dk == 128 && dm.dv == 128) return bf ? bwd_impl<bf16, 128, 128>(dm, args, a, s, events) : bwd_impl<float, 128, 128>(dm, args, a, s, events);
  if (dm.dk == 192 && dm.dv == 128) return bf ? bwd_impl<bf16, 192, 128>(dm, args, a, s, events) : bwd_impl<float, 192, 128>(dm, args, a, s, events);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Dense causal attention backward (the baseline's backward): the window
// branch's kernels with a window over every key and unit gates.
//   D = <dO, O> per row (O as the forward stored it), dq from the
//   query-tile kernel, dK/dV from the key-stationary window kernel.
// ---------------------------------------------------------------------------
template <typename T, int DV>
__global__ __launch_bounds__(256) void k_dense_rowterms(Dims dm, const T* __restrict__ o, const T* __restrict__ d_o,
                                                        const float* __restrict__ lse, float* __restrict__ Dc,
                                                        float* __restrict__ lse3, float* __restrict__ gates) {
  constexpr int LPR = DV / 4, RPW = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t BTH = (size_t)dm.B * dm.T * dm.Hq;
  const size_t row = ((size_t)blockIdx.x * 4 + wave) * RPW + lane / LPR;
  const int f = (lane % LPR) * 4;
  const bool live = row < BTH;
  const size_t rr = live ? row : 0;
  float d[4], x[4];
  load4(d_o + rr * DV + f, d);
  load4(o + rr * DV + f, x);
  float v = d[0] * x[0] + d[1] * x[1] + d[2] * x[2] + d[3] * x[3];
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if (!live || lane % LPR != 0) return;
  Dc[2 * BTH + row] = v;
  lse3[2 * BTH + row] = lse[row];
#pragma unroll
  for (int c = 0; c < 3; ++c) gates[row * 3 + c] = 1.f;
}

struct DenseBwdWs {
  float *gates, *Dc, *lse3;
  void* fkv;
};

static size_t dense_bwd_carve(const Dims& dm, void* ws, DenseBwdWs* w) {
  char* base = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t bytes) { void* r = base ? base + off : nullptr; off += al256(bytes); return r; };
  const size_t BTH = (size_t)dm.B * dm.T * dm.Hq, es = dm.io == IO_BF16 ? 2 : 4;
  w->gates = (float*)take(BTH * 3 * 4);
  w->Dc = (float*)take(3 * BTH * 4);
  w->lse3 = (float*)take(3 * BTH * 4);
  w->fkv = take(frag_tiles_elems(dm, dm.T, bwd_tile_ins(dm)) * es);
  return off;
}

size_t dense_bwd_ws_bytes(const Dims& dm) {
  DenseBwdWs w;
  return dense_bwd_carve(dm, nullptr, &w);
}

template <typename T, int DK, int DV>
static hipError_t dense_bwd_impl(Dims dm, const nsa_dense_bwd_args* args, void* ws, hipStream_t s) {
  if constexpr (!dq_tiled_fits<T, DK, DV>()) {
    return hipErrorInvalidValue;
  } else {
    dm.w = dm.T;
    DenseBwdWs w;
    dense_bwd_carve(dm, ws, &w);
    BwdArgs a{};
    a.q = args->q; a.k = args->k; a.v = args->v; a.d_o = args->d_o;
    a.ks = a.kw = args->k; a.vs = a.vw = args->v;
    a.lse = w.lse3;
    a.dq = (float*)args->dq;
    a.dk = a.dks = a.dkw = (float*)args->dk;
    a.dv = a.dvs = a.dvw = (float*)args->dv;
    a.w.gates = w.gates; a.w.Dc = w.Dc; a.w.fkv = w.fkv;
    a.fkv_win = w.fkv;
    hipError_t e;
    const size_t BTH = (size_t)dm.B * dm.T * dm.Hq;
    const size_t per_block = 4 * (64 / (DV / 4));
    k_dense_rowterms<T, DV><<<(unsigned)((BTH + per_block - 1) / per_block), 256, 0, s>>>(
        dm, (const T*)args->o, (const T*)args->d_o, (const float*)args->lse, w.Dc, w.lse3, w.gates);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int ti = bwd_tile_ins(dm);
    const int n1 = 2 * DK / 32, n2 = n1 + 2 * DV / 32;
    if ((e = launch_frag_pack(dm, DK, dm.T, a.k, w.fkv, ti, 0, false, s)) != hipSuccess ||
        (e = launch_frag_pack(dm, DV, dm.T, a.v, w.fkv, ti, n1, false, s)) != hipSuccess ||
        (e = launch_frag_pack(dm, DK, dm.T, a.k, w.fkv, ti, n2, true, s)) != hipSuccess)
      return e;
    if ((e = launch_dq_tiled<T, DK, DV, 4>(dm, a, s)) != hipSuccess) return e;
    const size_t klds = kv_lds<T, DK, DV>();
    if (klds > 64 * 1024)
      hipFuncSetAttribute((const void*)k_bwd_kv<T, DK, DV, KV_WIN>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)klds);
    k_bwd_kv<T, DK, DV, KV_WIN><<<dm.B * dm.Hkv * ((dm.T + 63) / 64), 256, klds, s>>>(dm, a);
    return hipGetLastError();
  }
}

bool dense_bwd_supported(const Dims& dm) {
  const bool bf = dm.io == IO_BF16;
  if (dm.dk == 64 && dm.dv == 64) return bf ? dq_tiled_fits<bf16, 64, 64>() : dq_tiled_fits<float, 64, 64>();
  if (dm.dk == 128 && dm.dv == 128) return bf ? dq_tiled_fits<bf16, 128, 128>() : dq_tiled_fits<float, 128, 128>();
  if (dm.dk == 192 && dm.dv == 128) return bf ? dq_tiled_fits<bf16, 192, 128>() : dq_tiled_fits<float, 192, 128>();
  return false;
}

hipError_t launch_dense_bwd(const Dims& dm, const nsa_dense_bwd_args* a, void* ws, hipStream_t s) {
  const bool bf = dm.io == IO_BF16;
  if (dm.dk == 64 && dm.dv == 64) return bf ? dense_bwd_impl<bf16, 64, 64>(dm, a, ws, s) : dense_bwd_impl<float, 64, 64>(dm, a, ws, s);
  if (dm.dk == 128 && dm.dv == 128) return bf ? dense_bwd_impl<bf16, 128, 128>(dm, a, ws, s) : dense_bwd_impl<float, 128, 128>(dm, a, ws, s);
  if (dm.dk == 192 && dm.dv == 128) return bf ? dense_bwd_impl<bf16, 192, 128>(dm, a, ws, s) : dense_bwd_impl<float, 192, 128>(dm, a, ws, s);
  return hipErrorInvalidValue;
}

}  // namespace nsa
