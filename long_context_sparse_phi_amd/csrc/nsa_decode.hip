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
// All caches are stored [key][Hkv][feature].  A wave reads each 32-key tile of
// its KV head as whole rows (64 lanes x 16 contiguous bytes per load, the
// request pattern that streams at full rate) into registers, one tile ahead,
// then writes it to LDS: keys row-major with XOR-swizzled chunks, values
// transposed ([feature][key]) so both MFMA operands are single 16-byte reads.
#include "../../include/nsa.h"
#include "nsa_common.hpp"
#include "nsa_kernels.hpp"
#include "nsa_tiles.hpp"

namespace nsa {

constexpr int kDecCK = 256;     // compressed blocks per chunk (one wave)
constexpr int kDecTPC = kDecCK / 32;
constexpr int kDecWinChunk = 64;
// tiles in flight per wave (one wave per SIMD; the ring takes most registers)
template <int DK, int DV> constexpr int dec_depth() { return DK + DV >= 320 ? 3 : 4; }

// Launch plan for the cache capacity S (grid sizes, workspace layout); every
// sequence then works within its own length (DecSeq).
struct DecPlan {
  int S, t, ncmp, nc, cpw, nb, jstep, nis, niw, ni, wlen, ws0;
};

static DecPlan dec_plan(const Dims& dm) {
  DecPlan p;
  p.S = dm.T;
  p.t = dm.T - 1;
  p.ncmp = dm.ncmp;
  p.nc = (dm.ncmp + kDecCK - 1) / kDecCK;
  // chunks per wave: about one wave per SIMD over the whole batch
  const long long chunks = (long long)dm.B * dm.Hkv * p.nc;
  p.cpw = 1;
  while (p.nc % (2 * p.cpw) == 0 && chunks / (2 * p.cpw) >= 1024) p.cpw *= 2;
  p.nb = (31 * dm.d + dm.l - 1) / dm.ls + 1;
  p.jstep = 32 * dm.d / dm.ls;
  p.nis = dm.n;
  p.wlen = dm.w < dm.T ? dm.w : dm.T;
  p.ws0 = dm.T - p.wlen;
  p.niw = (p.wlen + kDecWinChunk - 1) / kDecWinChunk;
  p.ni = p.nis + p.niw;
  return p;
}

struct DecBufs {
  float* part_o;    // [B,Hkv,nc,16,dv]
  float* part_ml;   // [B,Hkv,nc,16,2]
  float* part_ps;   // [B,Hkv,nc,TPC,nb,16] remapped scores, relative to the tile's running max
  float* part_tm;   // [B,Hkv,nc,TPC,16] running max (log2 units) after each tile
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
  b->part_tm = (float*)take(BG * p.nc * 16 * kDecTPC * 4);
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
  const int* lens;    // optional [B] tokens per sequence (NULL: S each)
  const void* kwcache;  // window branch's caches (the same as kcache, vcache
  const void* vwcache;  // unless each branch has its own keys and values)
  GateMlp gmlp;         // gate MLP first layer and biases (dm.Cg > 0)
  DecBufs w;
};

// Extent of sequence b: S tokens (clamped into [1, capacity]), query at t,
// ncmp complete compressed blocks, nsel selection blocks, the window's first
// token ws0 and its 64-token chunk count niw.
struct DecSeq {
  int S, t, ncmp, nsel, ws0, niw;
};

__device__ __forceinline__ DecSeq dec_seq(const Dims& dm, const DecArgs& a, int b) {
  DecSeq q;
  q.S = a.lens ? min(max(a.lens[b], 1), dm.T) : dm.T;
  q.t = q.S - 1;
  q.ncmp = q.S < dm.l ? 0 : (q.S - dm.l) / dm.d + 1;
  q.nsel = (q.S + dm.ls - 1) / dm.ls;
  const int wlen = min(dm.w, q.S);
  q.ws0 = q.S - wlen;
  q.niw = (wlen + kDecWinChunk - 1) / kDecWinChunk;
  return q;
}

// 32-key tile of one KV head: global -> registers (gload, one tile ahead of
// the compute) -> LDS (lstore).  Keys: 32 rows x DK, chunks swizzled by
// kchunk_off.  Values: V^T [DV][kVS]; a lane moves 4 consecutive key rows x 8
// features and writes them as 8-byte columns.  Lanes vary the feature chunk
// fastest within groups of 4, then the row quad, which spreads both the
// global requests (64 contiguous bytes per lane quad) and the LDS banks.
template <typename T, int DK, int DV>
struct DecTile {
  static constexpr int kVS = 40;                     // V^T row stride (elements)
  static constexpr int KCH = 32 * DK / 8 / 64;       // key chunks per lane
  static constexpr int VTK = DV / 64;                // value tasks (4 rows x 8 features) per lane
  static constexpr size_t kElems = (size_t)32 * DK;
  static constexpr size_t elems = kElems + (size_t)DV * kVS;
  Frag8<T> kr[KCH];
  Frag8<T> vr[VTK][4];

  __device__ __forceinline__ void gload(const T* kbase, const T* vbase, size_t kstride, size_t vstride, int key0,
                                        int klim, int lane) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int i = lane + 64 * c, row = i / (DK / 8), c8 = i % (DK / 8);
      kr[c] = load_frag(kbase + (size_t)min(key0 + row, klim - 1) * kstride + c8 * 8);
    }
#pragma unroll
    for (int c = 0; c < VTK; ++c) {
      const int u = lane + 64 * c, c8 = (u & 3) + 4 * (u >> 5), rq = (u >> 2) & 7;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        vr[c][k] = load_frag(vbase + (size_t)min(key0 + 4 * rq + k, klim - 1) * vstride + c8 * 8);
    }
  }
  __device__ __forceinline__ void lstore(T* tile, int lane) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int i = lane + 64 * c, row = i / (DK / 8), c8 = i % (DK / 8);
      *reinterpret_cast<Frag8<T>*>(tile + kchunk_off<DK>(row, c8)) = kr[c];
    }
    T* vt = tile + kElems;
#pragma unroll
    for (int c = 0; c < VTK; ++c) {
      const int u = lane + 64 * c, c8 = (u & 3) + 4 * (u >> 5), rq = (u >> 2) & 7;
      store_cols4x8(vt + (c8 * 8) * kVS + 4 * rq, kVS, vr[c]);
    }
  }
  // S^T = K Q^T for the tile's permuted key rows (two 16-key sub-tiles)
  static __device__ __forceinline__ void scores(f32x4 (&s)[2], const T* tile, const Frag8<T> (&qf)[DK / 32],
                                                int krow, int qd) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      Frag8<T> kf[DK / 32];
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
        kf[ks] = *reinterpret_cast<const Frag8<T>*>(tile + kchunk_off<DK>(krow + sub * 4, ks * 4 + qd));
      s[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) mma(s[sub], kf[ks], qf[ks]);
    }
  }
  // A operand of O^T += V^T P^T: feature dt*16 + c16, keys 8*qd .. 8*qd+7
  static __device__ __forceinline__ Frag8<T> vfrag(const T* tile, int dt, int c16, int qd) {
    return *reinterpret_cast<const Frag8<T>*>(tile + kElems + (dt * 16 + c16) * kVS + qd * 8);
  }
};

// Chunks of CK compressed keys, one pass with an online softmax: per tile the
// scores, the running per-head maximum, P V, and the remapped block scores
// relative to that running maximum, stored with it; the combine scales each
// tile's scores by exp2(max - lse).  A wave streams pl.cpw consecutive chunks
// of one (sequence, KV head) through a single ring of register tiles, so the
// ring stays full across chunk boundaries; each chunk's softmax state is
// written when its last tile is done.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(64, 1) void k_dec_cmp(Dims dm, DecArgs a, DecPlan pl) {
  using Tile = DecTile<T, DK, DV>;
  __shared__ __align__(16) T tile[Tile::elems];
  const int lane = threadIdx.x, c16 = lane & 15, qd = lane >> 4;
  const int wpb = pl.nc / pl.cpw;
  const int c0 = (blockIdx.x % wpb) * pl.cpw, bg = blockIdx.x / wpb;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int ncmp = dec_seq(dm, a, b).ncmp;
  const int k0 = c0 * kDecCK, k1 = min(k0 + pl.cpw * kDecCK, ncmp);
  const int ntile = k1 > k0 ? (k1 - k0 + 31) / 32 : 0;
  const bool cv = c16 < dm.G;
  Frag8<T> qf[DK / 32];
  {
    const T* qp = (const T*)a.q + ((size_t)b * dm.Hq + g * dm.G + (cv ? c16 : 0)) * DK + qd * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qf[ks] = cv ? load_frag(qp + ks * 32) : zero_frag<T>();
  }
  Frag8<T> wf[2];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = remap_weight(qd * 8 + e, jt * 16 + c16, dm.l, dm.d, dm.ls);
    wf[jt] = to_frag<T>(w);
  }
  const float sc2 = dm.scale * kLog2e;
  const size_t kstride = (size_t)dm.Hkv * DK, vstride = (size_t)dm.Hkv * DV;
  const T* kbase = (const T*)a.kc + ((size_t)b * a.cap * dm.Hkv + g) * DK;
  const T* vbase = (const T*)a.vc + ((size_t)b * a.cap * dm.Hkv + g) * DV;
  const int krow = (c16 >> 2) * 8 + (c16 & 3);
  f32x4 oacc[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f;
  // softmax state of chunk c: maximum, sum and unnormalised P V; then reset
  auto finish_chunk = [&](int c) {
    float l = lsum + xor16f(lsum, lane);
    l += xor32f(l, lane);
    const size_t hb = ((size_t)bg * pl.nc + c) * 16 + c16;
    if (qd == 0) {
      a.w.part_ml[hb * 2 + 0] = m;
      a.w.part_ml[hb * 2 + 1] = l;
    }
    float* op = a.w.part_o + hb * DV + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      store4(op + dt * 16, oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
      oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    m = kNegInf;
    lsum = 0.f;
  };
  auto compute = [&](int i) {
    const int kt = k0 + 32 * i;
    const int c = c0 + i / kDecTPC, ti = i % kDecTPC;
    float* ps = a.w.part_ps + (((size_t)bg * pl.nc + c) * kDecTPC + ti) * pl.nb * 16;
    float* tm = a.w.part_tm + (((size_t)bg * pl.nc + c) * kDecTPC + ti) * 16;
    f32x4 s[2];
    Tile::scores(s, tile, qf, krow, qd);
    float v[8], mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = (kt + qd * 8 + e < k1) ? s[e >> 2][e & 3] * sc2 : kNegInf;
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
    lsum = lsum * alpha + psum;
    m = mn;
    if (qd == 0) tm[c16] = mn;
    const Frag8<T> pf = to_frag<T>(p);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      oacc[dt] *= alpha;
      mma(oacc[dt], Tile::vfrag(tile, dt, c16, qd), pf);
    }
    Frag8<T> phi = pf, plo;
    if constexpr (sizeof(T) == 2) split_bf16(p, phi, plo);
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      if (jt * 16 >= pl.nb) break;
      f32x4 cr = f32x4{0.f, 0.f, 0.f, 0.f};
      mma(cr, phi, wf[jt]);
      if constexpr (sizeof(T) == 2) mma(cr, plo, wf[jt]);
      const int jj = jt * 16 + c16;
      if (jj < pl.nb) store4(ps + (size_t)jj * 16 + qd * 4, cr[0], cr[1], cr[2], cr[3]);
    }
    if (ti == kDecTPC - 1 || i == ntile - 1) finish_chunk(c);
  };
  // a ring of DEPTH tiles in flight in registers while the current one is
  // computed from LDS (one wave per SIMD, most of its registers hold loads)
  constexpr int DEPTH = dec_depth<DK, DV>();
  auto step = [&](Tile& cur, int i) {
    __syncthreads();
    cur.lstore(tile, lane);
    __syncthreads();
    if (i + DEPTH < ntile) cur.gload(kbase, vbase, kstride, vstride, k0 + 32 * (i + DEPTH), ncmp, lane);
    compute(i);
  };
  Tile ring[DEPTH];
#pragma unroll
  for (int r = 0; r < DEPTH; ++r)
    if (r < ntile) ring[r].gload(kbase, vbase, kstride, vstride, k0 + 32 * r, ncmp, lane);
  for (int i = 0; i < ntile; i += DEPTH) {
#pragma unroll
    for (int r = 0; r < DEPTH; ++r)
      if (i + r < ntile) step(ring[r], i + r);
  }
  // chunks past the sequence's compressed blocks hold an empty state
  for (int c = c0 + (ntile + kDecTPC - 1) / kDecTPC; c < c0 + pl.cpw; ++c) finish_chunk(c);
}

// Element i of an I/O tensor as float.
__device__ __forceinline__ float load_elem(const void* p, int io, size_t i) {
  return io == IO_BF16 ? (float)((const bf16*)p)[i] : ((const float*)p)[i];
}

// Length of the combine's LDS score row (it later holds the gate input).
static __host__ __device__ int comb_row_len(const Dims& dm) {
  return ((dm.nsel > dm.C ? dm.nsel : dm.C) + 3) & ~3;
}

// One workgroup (1024 threads) per (sequence, KV head): per-head log-sum-exp
// of the compressed branch, per-chunk scales, block scores and top-n.
__global__ __launch_bounds__(1024) void k_dec_combine(Dims dm, DecArgs a, DecPlan pl) {
  extern __shared__ float smem[];
  float* row = smem;                          // [nsel] block scores
  float* scl = row + comb_row_len(dm);        // [nc][16]
  float* lse2 = scl + pl.nc * 16;             // [16]
  float* mls = lse2 + 16;                     // [nc][16] chunk maxima
  float* lsl = mls + pl.nc * 16;              // [nc][16] chunk sums
  int* tsh = (int*)(lsl + pl.nc * 16);        // [256 + 16 + 4] top-n scratch
  float* ghid = (float*)(tsh + 256 + 16 + 4); // [Cg] gate MLP hidden layer
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bg = blockIdx.x, b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int G = dm.G;
  const DecSeq sq = dec_seq(dm, a, b);
  // gate inputs of head `wave`, requested after the chunk states and used at the end
  float gx[4], gw[4][3];
  auto gate_load = [&](int k0) {
    const int h = g * G + min(wave, G - 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u * 64 + lane;
      gx[u] = k < dm.C ? load_elem(a.x, dm.io, (size_t)b * dm.C + k) : 0.f;
#pragma unroll
      for (int c = 0; c < 3; ++c) gw[u][c] = k < dm.C ? load_elem(a.wg, dm.io, ((size_t)k * dm.Hq + h) * 3 + c) : 0.f;
    }
  };
  for (int i = tid; i < pl.nc * 16; i += 1024) {
    const size_t hb = (size_t)bg * pl.nc * 16 + i;
    mls[i] = a.w.part_ml[hb * 2];
    lsl[i] = a.w.part_ml[hb * 2 + 1];
  }
  if (dm.Cg == 0) gate_load(0);
  __syncthreads();
  // per-head log-sum-exp: wave h reduces head h over the chunks
  {
    const int h = wave;
    float M = kNegInf;
    for (int c = lane; c < pl.nc; c += 64) M = fmaxf(M, mls[c * 16 + h]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float Mr = M == kNegInf ? 0.f : M;
    float L = 0.f;
    for (int c = lane; c < pl.nc; c += 64) L += lsl[c * 16 + h] * fast_exp2(mls[c * 16 + h] - Mr);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    if (lane == 0) {
      const float l2 = M == kNegInf ? kNegInf : M + __log2f(L);
      lse2[h] = l2;
      if (h < G) a.w.lse_cmp[(size_t)b * dm.Hq + g * G + h] = l2;
    }
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
  const int ntiles = (sq.ncmp + 31) / 32;
  for (int j = tid; j < dm.nsel; j += 1024) {
    float val = 0.f;
    int klo = j - pl.nb + 1;
    klo = klo <= 0 ? 0 : (klo + pl.jstep - 1) / pl.jstep;
    const int khi = j < sq.nsel ? min(j / pl.jstep, ntiles - 1) : -1;
    // at most a few tiles touch a block; all their loads are issued together
    for (int kb = klo; kb <= khi; kb += 2) {
      float x[2][16], mt[2][16];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int kg = kb + q;
        if (kg > khi) break;
        const int c = kg / kDecTPC, i = kg % kDecTPC, jj = j - kg * pl.jstep;
        const float* ps = a.w.part_ps + ((((size_t)bg * pl.nc + c) * kDecTPC + i) * pl.nb + jj) * 16;
        const float* tm = a.w.part_tm + (((size_t)bg * pl.nc + c) * kDecTPC + i) * 16;
#pragma unroll
        for (int h4 = 0; h4 < 16; h4 += 4) {
          load4(ps + h4, x[q] + h4);
          load4(tm + h4, mt[q] + h4);
        }
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (kb + q > khi) break;
#pragma unroll
        for (int h = 0; h < 16; ++h)
          if (h < G && mt[q][h] != kNegInf && lse2[h] != kNegInf) val += x[q][h] * fast_exp2(mt[q][h] - lse2[h]);
      }
    }
    row[j] = val;
  }
  __syncthreads();
  if (a.p_slc)
    for (int j = tid; j < dm.nsel; j += 1024) a.p_slc[(size_t)bg * dm.nsel + j] = row[j];
  __syncthreads();
  block_topn<16>(row, sq.t, dm.ls, dm.n, a.w.idx + (size_t)bg * dm.n, tsh, tid);
  // gate MLP: this sequence's hidden layer gelu(x w1 + b1) in LDS, then the
  // output layer by the waves below over it
  if (dm.Cg > 0) {
    float* gx_s = row;   // the gate input of sequence b (the score row is no longer needed)
    __syncthreads();
    for (int k = tid; k < dm.C; k += 1024) gx_s[k] = load_elem(a.x, dm.io, (size_t)b * dm.C + k);
    __syncthreads();
    for (int j = tid; j < dm.Cg; j += 1024) {
      float acc = load_elem(a.gmlp.b1, dm.io, j);
#pragma unroll 8
      for (int k = 0; k < dm.C; ++k) acc = fmaf(gx_s[k], load_elem(a.gmlp.w1, dm.io, (size_t)k * dm.Cg + j), acc);
      ghid[j] = 0.5f * acc * (1.f + erff(acc * 0.70710678118654752f));
    }
    __syncthreads();
    if (wave < G) {
      const int h = g * G + wave;
      float z[3] = {0.f, 0.f, 0.f};
      for (int k = lane; k < dm.Cg; k += 64) {
#pragma unroll
        for (int c = 0; c < 3; ++c) z[c] = fmaf(ghid[k], load_elem(a.wg, dm.io, ((size_t)k * dm.Hq + h) * 3 + c), z[c]);
      }
#pragma unroll
      for (int c = 0; c < 3; ++c) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) z[c] += __shfl_xor(z[c], off);
      }
      if (lane < 3) {
        const float zz = (lane == 0 ? z[0] : (lane == 1 ? z[1] : z[2])) + load_elem(a.gmlp.b2, dm.io, (size_t)h * 3 + lane);
        a.w.gates[((size_t)b * dm.Hq + h) * 3 + lane] = 1.f / (1.f + expf(-zz));
      }
    }
    return;
  }
  // gates of the group's heads: wave h, lanes over the gate input, the three
  // branches together; the first 256 inputs were loaded at the start
  if (wave < G) {
    const int h = g * G + wave;
    float z[3] = {0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < dm.C; k0 += 4 * 64) {
      if (k0 > 0) gate_load(k0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 3; ++c) z[c] += gx[u] * gw[u][c];
    }
#pragma unroll
    for (int c = 0; c < 3; ++c) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) z[c] += __shfl_xor(z[c], off);
    }
    if (lane < 3) {
      const float zz = lane == 0 ? z[0] : (lane == 1 ? z[1] : z[2]);
      a.w.gates[((size_t)b * dm.Hq + h) * 3 + lane] = 1.f / (1.f + expf(-zz));
    }
  }
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(64) void k_dec_sw(Dims dm, DecArgs a, DecPlan pl) {
  using Tile = DecTile<T, DK, DV>;
  __shared__ __align__(16) T tile[Tile::elems];
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
  // key range of this work item: one selected block or one window chunk
  const DecSeq sq = dec_seq(dm, a, b);
  int r0 = 0, r1 = 0;
  if (it < pl.nis) {
    const int j = it < dm.n ? a.w.idx[(size_t)bg * dm.n + it] : -1;
    if (j >= 0) { r0 = j * dm.ls; r1 = min((j + 1) * dm.ls, sq.S); }
  } else if (it - pl.nis < sq.niw) {
    r0 = sq.ws0 + (it - pl.nis) * kDecWinChunk;
    r1 = min(r0 + kDecWinChunk, sq.S);
  }
  const int kt0 = r0 & ~31;
  const int ntile = r1 > r0 ? (r1 - kt0 + 31) / 32 : 0;
  const float sc2 = dm.scale * kLog2e;
  const size_t kstride = (size_t)dm.Hkv * DK, vstride = (size_t)dm.Hkv * DV;
  const bool win_item = it >= pl.nis;
  const T* kbase = (const T*)(win_item ? a.kwcache : a.kcache) + ((size_t)b * pl.S * dm.Hkv + g) * DK;
  const T* vbase = (const T*)(win_item ? a.vwcache : a.vcache) + ((size_t)b * pl.S * dm.Hkv + g) * DV;
  const int krow = (c16 >> 2) * 8 + (c16 & 3);
  float m = kNegInf, ls = 0.f;
  f32x4 oacc[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int i) {
    const int kt = kt0 + 32 * i;
    f32x4 s[2];
    Tile::scores(s, tile, qf, krow, qd);
    float v[8], mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = kt + qd * 8 + e;
      v[e] = (key >= r0 && key < r1) ? s[e >> 2][e & 3] * sc2 : kNegInf;
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
    const Frag8<T> pf = to_frag<T>(p);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      oacc[dt] *= alpha;
      mma(oacc[dt], Tile::vfrag(tile, dt, c16, qd), pf);
    }
  };
  // a ring of two tiles in flight (a 64-token block or aligned window chunk
  // is two tiles, so all of it is requested up front)
  auto step = [&](Tile& cur, int i) {
    __syncthreads();
    cur.lstore(tile, lane);
    __syncthreads();
    if (i + 2 < ntile) cur.gload(kbase, vbase, kstride, vstride, kt0 + 32 * (i + 2), sq.S, lane);
    compute(i);
  };
  Tile ring[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
    if (r < ntile) ring[r].gload(kbase, vbase, kstride, vstride, kt0 + 32 * r, sq.S, lane);
  for (int i = 0; i < ntile; i += 2) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
      if (i + r < ntile) step(ring[r], i + r);
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
  // gates of the two heads (evaluated by the combine)
  if (tid < 6) {
    const int hh = h0 + tid / 3;
    gts[tid] = hh < G ? a.w.gates[((size_t)b * dm.Hq + g * G + hh) * 3 + tid % 3] : 0.f;
  }
  // selected / window merge scales exp2(m_i - M_branch) / L_branch: one wave
  // per (head, branch) with the lanes over the items
  for (int o = wave; o < 4; o += 4) {
    const int hh = h0 + o / 2, br = o % 2;
    const int i0 = br == 0 ? 0 : pl.nis, i1 = br == 0 ? pl.nis : pl.ni;
    float M = kNegInf;
    for (int i = i0 + lane; i < i1; i += 64) M = fmaxf(M, a.w.sw_ml[(((size_t)bg * pl.ni + i) * 16 + hh) * 2]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float Mr = M == kNegInf ? 0.f : M;
    float L = 0.f;
    for (int i = i0 + lane; i < i1; i += 64) {
      const size_t hb = ((size_t)bg * pl.ni + i) * 16 + hh;
      L += a.w.sw_ml[hb * 2 + 1] * fast_exp2(a.w.sw_ml[hb * 2] - Mr);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    for (int i = i0 + lane; i < i1; i += 64) {
      const float mi = a.w.sw_ml[(((size_t)bg * pl.ni + i) * 16 + hh) * 2];
      swscl[i * 2 + o / 2] = mi == kNegInf ? 0.f : fast_exp2(mi - Mr) * inv;
    }
    if (a.lse && hh < G && lane == 0) {
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
#pragma unroll 8
  for (int c = 0; c < pl.nc; ++c) oc += a.w.part_o[(((size_t)bg * pl.nc + c) * 16 + hh) * DV + e] * cscl[c * 2 + hl];
  float ob[2] = {0.f, 0.f};
#pragma unroll 8
  for (int it = 0; it < pl.nis; ++it)
    ob[0] += a.w.sw_o[(((size_t)bg * pl.ni + it) * 16 + hh) * DV + e] * swscl[it * 2 + hl];
#pragma unroll 8
  for (int it = pl.nis; it < pl.ni; ++it)
    ob[1] += a.w.sw_o[(((size_t)bg * pl.ni + it) * 16 + hh) * DV + e] * swscl[it * 2 + hl];
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
    k_dec_cmp<T, DK, DV><<<BG * (pl.nc / pl.cpw), 64, 0, s>>>(dm, a, pl);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark()) != hipSuccess) return e;
  {
    const size_t lds = (size_t)comb_row_len(dm) * 4 + (size_t)pl.nc * 16 * 4 * 3 + 16 * 4 + (256 + 16 + 4) * 4 +
                       (size_t)dm.Cg * 4;
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
  a.lens = args->seq_lens;
  a.gmlp = GateMlp{args->gate_mlp.w1, args->gate_mlp.b1, args->gate_mlp.b2};
  a.kwcache = args->k_win_cache ? args->k_win_cache : args->k_cache;
  a.vwcache = args->v_win_cache ? args->v_win_cache : args->v_cache;
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
