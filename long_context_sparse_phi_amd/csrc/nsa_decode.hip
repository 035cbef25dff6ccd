// Single-token decode step for gfx950.
//
// Decoding is bound by how many cached bytes one step must read (youleyou NSA
// page, 效率分析/解码速度: per step the compressed tokens, the n*l' selected
// tokens and the w window tokens of each KV group).  Every cached byte is read
// once, by many waves in parallel:
//   1. k_dec_cmp: the compressed cache of each (sequence, KV group) is split
//      into chunks of CK blocks; a wave computes the group's 16 head scores for
//      its chunk, its partial softmax state (max m, sum l, unnormalised P V)
//      and its per-head partial importance scores remapped onto selection
//      blocks (same remap MFMA as the prefill).
//   2. k_dec_combine: merges the chunks' softmax states into exact per-head
//      probabilities, sums the group's heads into the block scores and runs
//      top-n.
//   3. k_dec_sw: one selected block or one 64-token window chunk per wave,
//      each a partial softmax state.
//   4. k_dec_merge: evaluates the gates, merges the compressed chunks and the
//      selected and window partial states, and writes
//      o = g_cmp O_cmp + g_slc O_slc + g_win O_win.
// The raw caches are stored [key][feature]; the value operand of P V needs
// eight consecutive keys per lane, so each 32-key value tile passes through
// LDS and is read transposed.
#include "../../include/nsa.h"
#include "nsa_common.hpp"
#include "nsa_kernels.hpp"

namespace nsa {

constexpr int kDecCK = 256;     // compressed blocks per chunk (one wave)
constexpr int kDecTPC = kDecCK / 32;
constexpr int kDecSlcPer = 1;   // selected blocks per wave
constexpr int kDecWinChunk = 64;

struct DecPlan {
  int S, t, ncmp, nc, nb, jstep, nis, niw, ni, wlen, ws0;
};

static DecPlan dec_plan(const Dims& dm) {
  DecPlan p;
  p.S = dm.T;
  p.t = dm.T - 1;
  p.ncmp = dm.ncmp;
  p.nc = (dm.ncmp + kDecCK - 1) / kDecCK;
  p.nb = (31 * dm.d + dm.l - 1) / dm.ls + 1;
  p.jstep = 32 * dm.d / dm.ls;
  p.nis = (dm.n + kDecSlcPer - 1) / kDecSlcPer;
  p.wlen = dm.w < dm.T ? dm.w : dm.T;
  p.ws0 = dm.T - p.wlen;
  p.niw = (p.wlen + kDecWinChunk - 1) / kDecWinChunk;
  p.ni = p.nis + p.niw;
  return p;
}

struct DecBufs {
  float* part_o;    // [B,Hkv,nc,16,dv]
  float* part_ml;   // [B,Hkv,nc,16,2]
  float* part_ps;   // [B,Hkv,nc,TPC,nb,16]
  float* cmp_scl;   // [B,Hkv,nc,16] exp2(m_chunk - lse) per chunk and head
  float* lse_cmp;   // [B,Hq] (log2 units)
  float* gates;     // [B,Hq,3]
  int* idx;         // [B,Hkv,n]
  float* sw_o;      // [B,Hkv,ni,16,dv]
  float* sw_ml;     // [B,Hkv,ni,16,2]
};

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t dec_carve(const Dims& dm, void* ws, DecBufs* b) {
  const DecPlan p = dec_plan(dm);
  char* base = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t bytes) { void* r = base ? base + off : nullptr; off += al256(bytes); return r; };
  const size_t BG = (size_t)dm.B * dm.Hkv;
  b->part_o = (float*)take(BG * p.nc * 16 * dm.dv * 4);
  b->part_ml = (float*)take(BG * p.nc * 16 * 2 * 4);
  b->part_ps = (float*)take(BG * p.nc * 16 * kDecTPC * p.nb * 4);
  b->cmp_scl = (float*)take(BG * (p.nc > 0 ? p.nc : 1) * 16 * 4);
  b->lse_cmp = (float*)take((size_t)dm.B * dm.Hq * 4);
  b->gates = (float*)take((size_t)dm.B * dm.Hq * 3 * 4);
  b->idx = (int*)take(BG * dm.n * 4);
  b->sw_o = (float*)take(BG * p.ni * 16 * dm.dv * 4);
  b->sw_ml = (float*)take(BG * p.ni * 16 * 2 * 4);
  return off;
}

size_t decode_ws_bytes(const Dims& dm) {
  DecBufs b;
  return dec_carve(dm, nullptr, &b);
}

struct DecArgs {
  const void* q;      // [B,Hq,dk]
  const void* kcache; // [B,S,Hkv,dk]
  const void* vcache; // [B,S,Hkv,dv]
  const void* kc;     // [B,cap,Hkv,dk]
  const void* vc;     // [B,cap,Hkv,dv]
  int cap;
  const void* x;      // [B,C]
  const void* wg;     // [C,Hq,3]
  void* o;            // [B,Hq,dv]
  float* p_slc;       // optional [B,Hkv,nsel]
  float* lse;         // optional [3,B,Hq]
  void* o_branch;     // optional [3,B,Hq,dv]
  DecBufs w;
};

// Loads a 32-key x DV value tile (rows key0..key0+31, clamped to klim-1) of
// one KV head into LDS [32][DV+8] and returns after the wave can read it.
template <typename T, int DV>
__device__ __forceinline__ void stage_v_tile(T* vs, const T* vbase, size_t kstride, int key0, int klim, int lane) {
  constexpr int CH = DV / 8;             // 16-byte chunks per row
  for (int i = lane; i < 32 * CH; i += 64) {
    const int r = i / CH, c = i % CH;
    const int key = min(key0 + r, klim - 1);
    Frag8<T> f = load_frag(vbase + (size_t)key * kstride + c * 8);
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<bf16x8*>(vs + r * (DV + 8) + c * 8) = f.v;
    } else {
      *reinterpret_cast<f32x4*>(vs + r * (DV + 8) + c * 8) = f.lo;
      *reinterpret_cast<f32x4*>(vs + r * (DV + 8) + c * 8 + 4) = f.hi;
    }
  }
  __syncthreads();
}

// A operand of O^T += V^T P^T from the staged tile: row dv = dt*16 + c16,
// keys 8*qd .. 8*qd+7.
template <typename T, int DV>
__device__ __forceinline__ Frag8<T> vt_frag(const T* vs, int dt, int c16, int qd) {
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = to_f32(vs[(qd * 8 + e) * (DV + 8) + dt * 16 + c16]);
  return to_frag<T>(x);
}

template <typename T, int DK>
__device__ __forceinline__ void score_tile(f32x4 (&s)[2], const T* kbase, size_t kstride, int kt, int klim,
                                           const Frag8<T> (&qf)[DK / 32], int krow) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    s[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int key = min(kt + krow + sub * 4, klim - 1);
    const T* kp = kbase + (size_t)key * kstride;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) mma(s[sub], load_frag(kp + ks * 32), qf[ks]);
  }
}

template <typename T, int DK>
__device__ __forceinline__ void load_k_tile(Frag8<T> (&kf)[2][DK / 32], const T* kbase, size_t kstride, int kt,
                                            int klim, int krow) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const T* kp = kbase + (size_t)min(kt + krow + sub * 4, klim - 1) * kstride;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) kf[sub][ks] = load_frag(kp + ks * 32);
  }
}

template <typename T, int DK>
__device__ __forceinline__ void score_from(f32x4 (&s)[2], const Frag8<T> (&kf)[2][DK / 32],
                                           const Frag8<T> (&qf)[DK / 32]) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    s[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) mma(s[sub], kf[sub][ks], qf[ks]);
  }
}

// 32-key value tile in registers (row r = key, 8 features per chunk) and its LDS image.
template <typename T, int DV>
struct VTileRegs {
  static constexpr int CH = 32 * DV / 8 / 64;   // chunks per lane
  Frag8<T> r[CH];
  __device__ __forceinline__ void gload(const T* vbase, size_t kstride, int key0, int klim, int lane) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = lane + 64 * c, row = i / (DV / 8), c8 = i % (DV / 8);
      r[c] = load_frag(vbase + (size_t)min(key0 + row, klim - 1) * kstride + c8 * 8);
    }
  }
  __device__ __forceinline__ void lstore(T* vs, int lane) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = lane + 64 * c, row = i / (DV / 8), c8 = i % (DV / 8);
      *reinterpret_cast<Frag8<T>*>(vs + row * (DV + 8) + c8 * 8) = r[c];
    }
  }
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(64) void k_dec_cmp(Dims dm, DecArgs a, DecPlan pl) {
  extern __shared__ __align__(16) float smem[];
  float* sb = smem;                                   // [TPC][64][8] scores
  T* vs = (T*)(smem + kDecTPC * 64 * 8);              // [32][DV+8]
  const int lane = threadIdx.x, c16 = lane & 15, qd = lane >> 4;
  const int c = blockIdx.x % pl.nc, bg = blockIdx.x / pl.nc;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int k0 = c * kDecCK, k1 = min(k0 + kDecCK, pl.ncmp);
  const int ntile = (k1 - k0 + 31) / 32;
  const bool cv = c16 < dm.G;
  Frag8<T> qf[DK / 32];
  {
    const T* qp = (const T*)a.q + ((size_t)b * dm.Hq + g * dm.G + (cv ? c16 : 0)) * DK + qd * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qf[ks] = cv ? load_frag(qp + ks * 32) : zero_frag<T>();
  }
  const float sc2 = dm.scale * kLog2e;
  const size_t kstride = (size_t)dm.Hkv * DK, vstride = (size_t)dm.Hkv * DV;
  const T* kbase = (const T*)a.kc + ((size_t)b * a.cap * dm.Hkv + g) * DK + qd * 8;
  const T* vbase = (const T*)a.vc + ((size_t)b * a.cap * dm.Hkv + g) * DV;
  const int krow = (c16 >> 2) * 8 + (c16 & 3);
  // phase 1: scores of the chunk, two key tiles in flight
  float mloc = kNegInf;
  auto keep = [&](const f32x4 (&s)[2], int i) {
    const int kt = k0 + 32 * i;
    float* dst = sb + (i * 64 + lane) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = (kt + qd * 8 + e < k1) ? s[e >> 2][e & 3] * sc2 : kNegInf;
      dst[e] = v;
      mloc = fmaxf(mloc, v);
    }
  };
  {
    Frag8<T> ka[2][DK / 32], kb[2][DK / 32];
    load_k_tile<T, DK>(ka, kbase, kstride, k0, pl.ncmp, krow);
    for (int i = 0; i < ntile; i += 2) {
      if (i + 1 < ntile) load_k_tile<T, DK>(kb, kbase, kstride, k0 + 32 * (i + 1), pl.ncmp, krow);
      f32x4 s[2];
      score_from<T, DK>(s, ka, qf);
      keep(s, i);
      if (i + 2 < ntile) load_k_tile<T, DK>(ka, kbase, kstride, k0 + 32 * (i + 2), pl.ncmp, krow);
      if (i + 1 < ntile) {
        score_from<T, DK>(s, kb, qf);
        keep(s, i + 1);
      }
    }
  }
  mloc = fmaxf(mloc, xor16f(mloc, lane));
  mloc = fmaxf(mloc, xor32f(mloc, lane));
  const float mref = mloc == kNegInf ? 0.f : mloc;
  Frag8<T> wf[2];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = remap_weight(qd * 8 + e, jt * 16 + c16, dm.l, dm.d, dm.ls);
    wf[jt] = to_frag<T>(w);
  }
  f32x4 oacc[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  float* ps = a.w.part_ps + ((size_t)bg * pl.nc + c) * kDecTPC * pl.nb * 16;
  // phase 2: probabilities, P V and remapped scores; the next value tile is in flight
  VTileRegs<T, DV> vr;
  vr.gload(vbase, vstride, k0, pl.ncmp, lane);
  for (int i = 0; i < ntile; ++i) {
    __syncthreads();
    vr.lstore(vs, lane);
    __syncthreads();
    if (i + 1 < ntile) vr.gload(vbase, vstride, k0 + 32 * (i + 1), pl.ncmp, lane);
    float p[8];
    const float* src = sb + (i * 64 + lane) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) { p[e] = fast_exp2(src[e] - mref); lsum += p[e]; }
    Frag8<T> pf = to_frag<T>(p);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) mma(oacc[dt], vt_frag<T, DV>(vs, dt, c16, qd), pf);
    Frag8<T> phi = pf, plo;
    if constexpr (sizeof(T) == 2) split_bf16(p, phi, plo);
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      if (jt * 16 >= pl.nb) break;
      f32x4 cr = f32x4{0.f, 0.f, 0.f, 0.f};
      mma(cr, phi, wf[jt]);
      if constexpr (sizeof(T) == 2) mma(cr, plo, wf[jt]);
      const int jj = jt * 16 + c16;
      if (jj < pl.nb) store4(ps + ((size_t)i * pl.nb + jj) * 16 + qd * 4, cr[0], cr[1], cr[2], cr[3]);
    }
  }
  lsum += xor16f(lsum, lane);
  lsum += xor32f(lsum, lane);
  const size_t hb = ((size_t)bg * pl.nc + c) * 16 + c16;
  if (qd == 0) {
    a.w.part_ml[hb * 2 + 0] = mloc;
    a.w.part_ml[hb * 2 + 1] = lsum;
  }
  float* op = a.w.part_o + hb * DV + qd * 4;
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) store4(op + dt * 16, oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
}

// One workgroup (1024 threads) per (sequence, KV head): per-head log-sum-exp
// of the compressed branch, per-chunk scales, block scores and top-n.
__global__ __launch_bounds__(1024) void k_dec_combine(Dims dm, DecArgs a, DecPlan pl) {
  extern __shared__ float smem[];
  float* row = smem;                          // [nsel]
  float* scl = row + ((dm.nsel + 3) & ~3);    // [nc][16]
  float* lse2 = scl + pl.nc * 16;             // [16]
  float* mls = lse2 + 16;                     // [nc][16] chunk maxima
  float* lsl = mls + pl.nc * 16;              // [nc][16] chunk sums
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bg = blockIdx.x, b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int G = dm.G;
  for (int i = tid; i < pl.nc * 16; i += 1024) {
    const size_t hb = (size_t)bg * pl.nc * 16 + i;
    mls[i] = a.w.part_ml[hb * 2];
    lsl[i] = a.w.part_ml[hb * 2 + 1];
  }
  __syncthreads();
  if (tid < 16) {
    float M = kNegInf;
    for (int c = 0; c < pl.nc; ++c) M = fmaxf(M, mls[c * 16 + tid]);
    float L = 0.f;
    const float Mr = M == kNegInf ? 0.f : M;
    for (int c = 0; c < pl.nc; ++c) L += lsl[c * 16 + tid] * fast_exp2(mls[c * 16 + tid] - Mr);
    const float l2 = M == kNegInf ? kNegInf : M + __log2f(L);
    lse2[tid] = l2;
    if (tid < G) a.w.lse_cmp[(size_t)b * dm.Hq + g * G + tid] = l2;
  }
  __syncthreads();
  for (int i = tid; i < pl.nc * 16; i += 1024) {
    const float mc = mls[i], l2 = lse2[i % 16];
    const float v = (mc == kNegInf || l2 == kNegInf) ? 0.f : fast_exp2(mc - l2);
    scl[i] = v;
    a.w.cmp_scl[(size_t)bg * pl.nc * 16 + i] = v;
  }
  __syncthreads();
  // block scores: sum over heads of exact probabilities remapped to blocks
  const int ntiles = (pl.ncmp + 31) / 32;
  for (int j = tid; j < dm.nsel; j += 1024) {
    float val = 0.f;
    int klo = j - pl.nb + 1;
    klo = klo <= 0 ? 0 : (klo + pl.jstep - 1) / pl.jstep;
    const int khi = min(j / pl.jstep, ntiles - 1);
    for (int kg = klo; kg <= khi; ++kg) {
      const int c = kg / kDecTPC, i = kg % kDecTPC, jj = j - kg * pl.jstep;
      const float* ps = a.w.part_ps + ((((size_t)bg * pl.nc + c) * kDecTPC + i) * pl.nb + jj) * 16;
      for (int h4 = 0; h4 < G; h4 += 4) {
        float x[4];
        load4(ps + h4, x);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (h4 + r < G) val += x[r] * scl[c * 16 + h4 + r];
      }
    }
    row[j] = val;
  }
  __syncthreads();
  if (a.p_slc)
    for (int j = tid; j < dm.nsel; j += 1024) a.p_slc[(size_t)bg * dm.nsel + j] = row[j];
  __syncthreads();
  if (wave == 0) wave_topn(row, pl.t, dm.ls, dm.n, a.w.idx + (size_t)bg * dm.n, lane);
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(64) void k_dec_sw(Dims dm, DecArgs a, DecPlan pl) {
  __shared__ T vs[32 * (DV + 8)];
  const int lane = threadIdx.x, c16 = lane & 15, qd = lane >> 4;
  const int it = blockIdx.x % pl.ni, bg = blockIdx.x / pl.ni;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  const bool cv = c16 < dm.G;
  Frag8<T> qf[DK / 32];
  {
    const T* qp = (const T*)a.q + ((size_t)b * dm.Hq + g * dm.G + (cv ? c16 : 0)) * DK + qd * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qf[ks] = cv ? load_frag(qp + ks * 32) : zero_frag<T>();
  }
  // key ranges of this work item
  int r0[kDecSlcPer], r1[kDecSlcPer], nr = 0;
  if (it < pl.nis) {
    for (int s = 0; s < kDecSlcPer; ++s) {
      const int si = it * kDecSlcPer + s;
      const int j = si < dm.n ? a.w.idx[(size_t)bg * dm.n + si] : -1;
      if (j >= 0) { r0[nr] = j * dm.ls; r1[nr] = min((j + 1) * dm.ls, pl.S); ++nr; }
    }
  } else {
    const int wi = it - pl.nis;
    r0[0] = pl.ws0 + wi * kDecWinChunk;
    r1[0] = min(r0[0] + kDecWinChunk, pl.S);
    nr = 1;
  }
  const float sc2 = dm.scale * kLog2e;
  const size_t kstride = (size_t)dm.Hkv * DK, vstride = (size_t)dm.Hkv * DV;
  const T* kbase = (const T*)a.kcache + ((size_t)b * pl.S * dm.Hkv + g) * DK + qd * 8;
  const T* vbase = (const T*)a.vcache + ((size_t)b * pl.S * dm.Hkv + g) * DV;
  const int krow = (c16 >> 2) * 8 + (c16 & 3);
  float m = kNegInf, ls = 0.f;
  f32x4 oacc[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < nr; ++r) {
    for (int kt = r0[r]; kt < r1[r]; kt += 32) {
      f32x4 s[2];
      score_tile<T, DK>(s, kbase, kstride, kt, pl.S, qf, krow);
      __syncthreads();
      stage_v_tile<T, DV>(vs, vbase, vstride, kt, pl.S, lane);
      float v[8], mx = kNegInf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = (kt + qd * 8 + e < r1[r]) ? s[e >> 2][e & 3] * sc2 : kNegInf;
        mx = fmaxf(mx, v[e]);
      }
      mx = fmaxf(mx, xor16f(mx, lane));
      mx = fmaxf(mx, xor32f(mx, lane));
      const float mn = fmaxf(m, mx);
      const float mref = mn == kNegInf ? 0.f : mn;
      const float alpha = fast_exp2(m - mref);
      float p[8], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) { p[e] = fast_exp2(v[e] - mref); psum += p[e]; }
      ls = ls * alpha + psum;
      m = mn;
      Frag8<T> pf = to_frag<T>(p);
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) {
        oacc[dt] *= alpha;
        mma(oacc[dt], vt_frag<T, DV>(vs, dt, c16, qd), pf);
      }
    }
  }
  ls += xor16f(ls, lane);
  ls += xor32f(ls, lane);
  const size_t hb = ((size_t)bg * pl.ni + it) * 16 + c16;
  if (qd == 0) {
    a.w.sw_ml[hb * 2 + 0] = m;
    a.w.sw_ml[hb * 2 + 1] = ls;
  }
  float* op = a.w.sw_o + hb * DV + qd * 4;
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) store4(op + dt * 16, oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
}

// One workgroup per (sequence, KV head, pair of query heads): gates, merge of
// the compressed chunks and of the selected/window partial states, output.
template <typename T, int DV>
__global__ __launch_bounds__(256) void k_dec_merge(Dims dm, DecArgs a, DecPlan pl) {
  extern __shared__ float sm[];
  float* swscl = sm;                  // [ni][2]
  float* cscl = swscl + pl.ni * 2;    // [nc][2]
  float* gts = cscl + pl.nc * 2;      // [2][3]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hp = blockIdx.x % 8, bg = blockIdx.x / 8;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int G = dm.G;
  const int h0 = hp * 2;
  if (h0 >= G) return;
  // gates of the two heads: one wave per dot product
  for (int o = wave; o < 6; o += 4) {
    const int hh = h0 + o / 3, cc = o % 3;
    float z = 0.f;
    if (hh < G) {
      const int h = g * G + hh;
      for (int k = lane; k < dm.C; k += 64)
        z += to_f32(((const T*)a.x)[(size_t)b * dm.C + k]) * to_f32(((const T*)a.wg)[((size_t)k * dm.Hq + h) * 3 + cc]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
    if (lane == 0) gts[o] = 1.f / (1.f + expf(-z));
  }
  // selected / window merge scales: exp2(m_i - M_branch) / L_branch
  if (tid < 4) {
    const int hh = h0 + tid / 2, br = tid % 2;
    const int i0 = br == 0 ? 0 : pl.nis, i1 = br == 0 ? pl.nis : pl.ni;
    float M = kNegInf;
    for (int i = i0; i < i1; ++i) M = fmaxf(M, a.w.sw_ml[(((size_t)bg * pl.ni + i) * 16 + hh) * 2]);
    const float Mr = M == kNegInf ? 0.f : M;
    float L = 0.f;
    for (int i = i0; i < i1; ++i) {
      const size_t hb = ((size_t)bg * pl.ni + i) * 16 + hh;
      L += a.w.sw_ml[hb * 2 + 1] * fast_exp2(a.w.sw_ml[hb * 2] - Mr);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    for (int i = i0; i < i1; ++i) {
      const float mi = a.w.sw_ml[(((size_t)bg * pl.ni + i) * 16 + hh) * 2];
      swscl[i * 2 + tid / 2] = mi == kNegInf ? 0.f : fast_exp2(mi - Mr) * inv;
    }
    if (a.lse && hh < G) {
      const size_t rr = (size_t)b * dm.Hq + g * G + hh;
      a.lse[(size_t)(1 + br) * dm.B * dm.Hq + rr] = (M + __log2f(L)) * kLn2;
      if (br == 0) {
        const float l2 = a.w.lse_cmp[rr];
        a.lse[rr] = l2 == kNegInf ? kNegInf : l2 * kLn2;
      }
    }
  }
  for (int i = tid; i < pl.nc * 2; i += 256) cscl[i] = a.w.cmp_scl[((size_t)bg * pl.nc + i / 2) * 16 + h0 + i % 2];
  __syncthreads();
  const int hh = h0 + tid / DV, e = tid % DV;   // 2 heads x DV features (DV <= 128)
  if (tid >= 2 * DV || hh >= G) return;
  const int hl = hh - h0;
  float oc = 0.f;
  for (int c = 0; c < pl.nc; ++c) oc += a.w.part_o[(((size_t)bg * pl.nc + c) * 16 + hh) * DV + e] * cscl[c * 2 + hl];
  float ob[2] = {0.f, 0.f};
  for (int it = 0; it < pl.ni; ++it) {
    const float v = a.w.sw_o[(((size_t)bg * pl.ni + it) * 16 + hh) * DV + e] * swscl[it * 2 + hl];
    if (it < pl.nis) ob[0] += v; else ob[1] += v;
  }
  const size_t row = (size_t)b * dm.Hq + g * G + hh;
  const float o = gts[hl * 3 + 0] * oc + gts[hl * 3 + 1] * ob[0] + gts[hl * 3 + 2] * ob[1];
  ((T*)a.o)[row * DV + e] = from_f32<T>(o);
  if (a.o_branch) {
    const size_t plane = (size_t)dm.B * dm.Hq * DV;
    ((float*)a.o_branch)[row * DV + e] = oc;
    ((float*)a.o_branch)[plane + row * DV + e] = ob[0];
    ((float*)a.o_branch)[2 * plane + row * DV + e] = ob[1];
  }
}

template <typename T, int DK, int DV>
static hipError_t decode_impl(const Dims& dm, const DecArgs& a, const DecPlan& pl, hipStream_t s,
                              void* const* events) {
  int ei = 0;
  auto mark = [&]() { return events ? hipEventRecord((hipEvent_t)events[ei++], s) : hipSuccess; };
  hipError_t e;
  const int BG = dm.B * dm.Hkv;
  if ((e = mark()) != hipSuccess) return e;
  if (pl.nc > 0) {
    const size_t lds = (size_t)kDecTPC * 64 * 8 * 4 + 32 * (DV + 8) * sizeof(T);
    k_dec_cmp<T, DK, DV><<<BG * pl.nc, 64, lds, s>>>(dm, a, pl);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark()) != hipSuccess) return e;
  {
    const size_t lds = (((size_t)dm.nsel + 3) & ~(size_t)3) * 4 + (size_t)pl.nc * 16 * 4 * 3 + 16 * 4;
    if (lds > 64 * 1024)
      hipFuncSetAttribute((const void*)k_dec_combine, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    k_dec_combine<<<BG, 1024, lds, s>>>(dm, a, pl);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark()) != hipSuccess) return e;
  k_dec_sw<T, DK, DV><<<BG * pl.ni, 64, 0, s>>>(dm, a, pl);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_dec_merge<T, DV><<<BG * 8, 256, ((size_t)pl.ni * 2 + (size_t)pl.nc * 2 + 8) * sizeof(float), s>>>(dm, a, pl);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark();
}

hipError_t launch_decode(const Dims& dm, const nsa_decode_args* args, void* ws, hipStream_t s,
                         void* const* events) {
  DecArgs a;
  a.q = args->q; a.kcache = args->k_cache; a.vcache = args->v_cache;
  a.kc = args->k_cmp_cache; a.vc = args->v_cmp_cache; a.cap = args->cmp_cache_cap;
  a.x = args->x; a.wg = args->w_gate; a.o = args->o;
  a.p_slc = (float*)args->p_slc; a.lse = (float*)args->lse; a.o_branch = args->o_branch;
  dec_carve(dm, ws, &a.w);
  if (args->idx) a.w.idx = (int*)args->idx;
  const DecPlan pl = dec_plan(dm);
  const bool bf = dm.io == IO_BF16;
  if (dm.dk == 64 && dm.dv == 64) return bf ? decode_impl<bf16, 64, 64>(dm, a, pl, s, events) : decode_impl<float, 64, 64>(dm, a, pl, s, events);
  if (dm.dk == 128 && dm.dv == 128) return bf ? decode_impl<bf16, 128, 128>(dm, a, pl, s, events) : decode_impl<float, 128, 128>(dm, a, pl, s, events);
  if (dm.dk == 192 && dm.dv == 128) return bf ? decode_impl<bf16, 192, 128>(dm, a, pl, s, events) : decode_impl<float, 192, 128>(dm, a, pl, s, events);
  return hipErrorInvalidValue;
}

}  // namespace nsa
