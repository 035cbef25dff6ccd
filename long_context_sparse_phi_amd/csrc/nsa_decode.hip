// Single-token decode step for gfx950.
//
// Decoding is bound by how many cached bytes one step must read (youleyou NSA
// page, 效率分析/解码速度: per step the compressed tokens, the n*l' selected
// tokens and the w window tokens of each KV group).  Every cached byte is read
// once, by many waves in parallel:
//   1. k_dec_cmp: the compressed cache of each (sequence, KV group) is split
//      into chunks of CK blocks; a wave computes the group's 16 head scores for
//      its consecutive chunks, their partial softmax state (max m, sum l,
//      unnormalised P V) and the per-head partial importance scores of each
//      tile remapped onto selection blocks (same remap MFMA as the prefill).
//   2. k_dec_combine: merges the waves' softmax states into exact per-head
//      probabilities, sums the group's heads into the block scores and runs
//      top-n.
//   3. k_dec_sw: one selected block or one 64-token window chunk per wave,
//      each a partial softmax state.
//   4. k_dec_merge: evaluates the gates, merges the compressed states and the
//      selected and window partial states, and writes
//      o = g_cmp O_cmp + g_slc O_slc + g_win O_win.
// All caches are stored [key][Hkv][feature].  A wave reads each 32-key tile of
// its KV head as whole rows (64 lanes x 16 contiguous bytes per load, the
// request pattern that streams at full rate) into registers, one tile ahead,
// then writes it to LDS: keys row-major with XOR-swizzled chunks, values
// transposed ([feature][key]) so both MFMA operands are single 16-byte reads.
#include <mutex>

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
  int S, t, ncmp, nc, cpw, ns, nb, jstep, nis, niw, ni, wlen, ws0;
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
  p.ns = p.nc / p.cpw;   // softmax states per (sequence, KV head): one per wave
  p.nb = (31 * dm.d + dm.l - 1) / dm.ls + 1;
  p.jstep = 32 * dm.d / dm.ls;
  // work items of the selected/window pass: two selected blocks, or two
  // 64-token window chunks, each
  p.nis = (dm.n + 1) / 2;
  p.wlen = dm.w < dm.T ? dm.w : dm.T;
  p.ws0 = dm.T - p.wlen;
  p.niw = ((p.wlen + kDecWinChunk - 1) / kDecWinChunk + 1) / 2;
  p.ni = p.nis + p.niw;
  return p;
}

struct DecBufs {
  float* part_o;    // [B,Hkv,ns,16,dv] unnormalised P V of each wave's chunks
  float* part_ml;   // [B,Hkv,ns,16,2]
  float* part_ps;   // [B,Hkv,nc,TPC,nb,16] remapped scores, relative to the tile's running max
  float* part_tm;   // [B,Hkv,nc,TPC,16] running max (log2 units) after each tile
  float* cmp_scl;   // [B,Hkv,ns,16] exp2(m_wave - lse) per wave and head
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
  b->part_o = (float*)take(BG * p.ns * 16 * dm.dv * 4);
  b->part_ml = (float*)take(BG * p.ns * 16 * 2 * 4);
  b->part_ps = (float*)take(BG * p.nc * 16 * kDecTPC * p.nb * 4);
  b->part_tm = (float*)take(BG * p.nc * 16 * kDecTPC * 4);
  b->cmp_scl = (float*)take(BG * (p.ns > 0 ? p.ns : 1) * 16 * 4);
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

// Scratch of the allocation-free decode entry point: one copy per GPU,
// created with the code object and held until the process ends.  In host code
// `scratch` is only a stand-in for the symbol; its device address differs per
// GPU and comes from hipGetSymbolAddress with that GPU current.
static __device__ __align__(256) unsigned char scratch[NSA_DECODE_STATIC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per
// device and kept.
hipError_t decode_static_scratch(void** out) {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
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
// kchunk_off; load c moves rows 8*(c%4) .. +7, 8 consecutive 16-byte chunks
// of each (128 contiguous bytes per row).  Values: V^T [DV][kVS]; a lane
// moves 4 consecutive key rows x 8 features and writes them as 8-byte
// columns.  Lanes vary the feature chunk fastest within groups of 4, then the
// row quad, which spreads both the global requests (64 contiguous bytes per
// lane quad) and the LDS banks.  Addresses are a wave-uniform tile base plus
// a 24-bit row product per lane, so a load costs a few full-rate VALU
// operations.
template <typename T, int DK, int DV>
struct DecTile {
  static constexpr int kVS = 40;                     // V^T row stride (elements)
  static constexpr int KCH = 32 * DK / 8 / 64;       // key chunks per lane
  static constexpr int VTK = DV / 64;                // value tasks (4 rows x 8 features) per lane
  static constexpr size_t kElems = (size_t)32 * DK;
  static constexpr size_t elems = kElems + (size_t)DV * kVS;
  static_assert(DK % 64 == 0, "key rows are moved in groups of 8 chunks");
  Frag8<T> kr[KCH];
  Frag8<T> vr[VTK][4];
  static __device__ __forceinline__ int krow(int c, int lane) { return (c & 3) * 8 + (lane >> 3); }
  static __device__ __forceinline__ int kchunk(int c, int lane) { return (c >> 2) * 8 + (lane & 7); }

  // rows past klim - 1 (the tail of the last tile) read row klim - 1.  NT:
  // non-temporal loads, for data read once (the compressed cache streams
  // through once per step; the selected blocks and window chunks overlap)
  template <bool NT = false>
  __device__ __forceinline__ void gload(const T* kbase, const T* vbase, size_t kstride, size_t vstride, int key0,
                                        int klim, int lane) {
    auto ld = [](const T* p) {
      if constexpr (NT) return load_frag_nt(p);
      else return load_frag(p);
    };
    const T* kt = kbase + (size_t)key0 * kstride;
    const T* vt = vbase + (size_t)key0 * vstride;
    const int rmax = klim - 1 - key0;
#pragma unroll
    for (int c = 0; c < KCH; ++c)
      kr[c] = ld(kt + __umul24((unsigned)min(krow(c, lane), rmax), (unsigned)kstride) + kchunk(c, lane) * 8);
#pragma unroll
    for (int c = 0; c < VTK; ++c) {
      const int u = lane + 64 * c, c8 = (u & 3) + 4 * (u >> 5), rq = (u >> 2) & 7;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        vr[c][k] = ld(vt + __umul24((unsigned)min(4 * rq + k, rmax), (unsigned)vstride) + c8 * 8);
    }
  }
  __device__ __forceinline__ void lstore(T* tile, int lane) {
#pragma unroll
    for (int c = 0; c < KCH; ++c)
      *reinterpret_cast<Frag8<T>*>(tile + kchunk_off<DK>(krow(c, lane), kchunk(c, lane))) = kr[c];
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
// tile's scores by exp2(max - lse).  A wave takes pl.cpw consecutive chunks
// of one (sequence, KV head); each chunk streams through the ring of register
// tiles, one online softmax runs through all of them, and the wave writes its
// softmax state once, after its last chunk.  A chunk's per-tile block scores
// and reference maxima are kept in LDS and written after the chunk's loads
// (one round of the ring per chunk): global stores issued
// between the ring's loads would make the loads' completion count ambiguous,
// and every tile would then wait for all loads in flight.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(64, 1) void k_dec_cmp(Dims dm, DecArgs a, DecPlan pl) {
  using Tile = DecTile<T, DK, DV>;
  __shared__ __align__(16) T tile[Tile::elems];
  __shared__ __align__(16) float sps[kDecTPC * 32 * 16];   // [tile][block][head], nb <= 32
  __shared__ __align__(16) float stm[kDecTPC * 16];        // [tile][head]
  const int lane = threadIdx.x, c16 = lane & 15, qd = lane >> 4;
  const int wpb = pl.nc / pl.cpw;
  const int c0 = (blockIdx.x % wpb) * pl.cpw, bg = blockIdx.x / wpb;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int ncmp = dec_seq(dm, a, b).ncmp;
  const int k0 = c0 * kDecCK, k1 = min(k0 + pl.cpw * kDecCK, ncmp);
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
  // the tiles' block scores and maxima of chunk c (nt tiles)
  auto finish_chunk = [&](int c, int nt) {
    if (nt > 0) {
      __syncthreads();
      const size_t tb = ((size_t)bg * pl.nc + c) * kDecTPC;
      float* gps = a.w.part_ps + tb * pl.nb * 16;
      for (int e = lane * 4; e < nt * pl.nb * 16; e += 256)
        *reinterpret_cast<f32x4*>(gps + e) = *reinterpret_cast<const f32x4*>(sps + e);
      for (int e = lane * 4; e < nt * 16; e += 256)
        *reinterpret_cast<f32x4*>(a.w.part_tm + tb * 16 + e) = *reinterpret_cast<const f32x4*>(stm + e);
    }
  };
  // the softmax state of all of the wave's chunks (one online softmax runs
  // through them): maximum, sum and unnormalised P V
  auto finish_wave = [&]() {
    float l = lsum + xor16f(lsum, lane);
    l += xor32f(l, lane);
    const size_t hb = ((size_t)bg * pl.ns + blockIdx.x % wpb) * 16 + c16;
    if (qd == 0) {
      a.w.part_ml[hb * 2 + 0] = m;
      a.w.part_ml[hb * 2 + 1] = l;
    }
    float* op = a.w.part_o + hb * DV + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) store4(op + dt * 16, oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]);
  };
  // tile ti of the chunk starting at key kc0
  auto compute = [&](int kc0, int ti) {
    const int kt = kc0 + 32 * ti;
    float* ps = sps + ti * pl.nb * 16;
    float* tm = stm + ti * 16;
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
    // Lazy rescaling: a head's reference m moves only when the tile's maximum
    // exceeds it by more than 8 (so p <= 2^8), decided for the whole wave.
    // The tile's probabilities and remapped scores are relative to m, which
    // is what part_tm records.
    if (__builtin_amdgcn_ballot_w64(mx > m + 8.f) != 0) {
      const float mn = fmaxf(m, mx);
      const float alpha = mn == kNegInf ? 1.f : fast_exp2(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) oacc[dt] *= alpha;
      m = mn;
    }
    const float mref = m == kNegInf ? 0.f : m;
    float p[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { p[e] = fast_exp2(v[e] - mref); psum += p[e]; }
    lsum += psum;
    if (qd == 0) tm[c16] = m;
    const Frag8<T> pf = to_frag<T>(p);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) mma(oacc[dt], Tile::vfrag(tile, dt, c16, qd), pf);
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
  };
  // Each chunk streams through a ring of DEPTH register tiles, computed from
  // LDS one at a time (one wave per SIMD, most of its registers hold loads).
  // Every full round of DEPTH tiles issues DEPTH tiles' loads (past the
  // chunk's last tile they re-read it), so the wait for a tile covers that
  // tile's loads only; the chunk's global stores follow its ring and are
  // complete before the next chunk's loads are issued.  The cache is read
  // once per step, with non-temporal loads.
  constexpr int DEPTH = dec_depth<DK, DV>();
  Tile ring[DEPTH];
  for (int cc = 0; cc < pl.cpw; ++cc) {
    const int c = c0 + cc, kc0 = k0 + cc * kDecCK;
    const int nt = kc0 < k1 ? min(kDecTPC, (k1 - kc0 + 31) / 32) : 0;
    if (nt > 0) {
      auto tkey = [&](int ti) { return kc0 + 32 * min(ti, nt - 1); };
      auto step = [&](Tile& cur, int ti, bool refill) {
        __syncthreads();
        cur.lstore(tile, lane);
        __syncthreads();
        if (refill) cur.template gload<true>(kbase, vbase, kstride, vstride, tkey(ti + DEPTH), ncmp, lane);
        compute(kc0, ti);
      };
#pragma unroll
      for (int r = 0; r < DEPTH; ++r) ring[r].template gload<true>(kbase, vbase, kstride, vstride, tkey(r), ncmp, lane);
      int i0 = 0;
      for (; i0 + DEPTH <= nt; i0 += DEPTH) {
#pragma unroll
        for (int r = 0; r < DEPTH; ++r) step(ring[r], i0 + r, true);
      }
#pragma unroll
      for (int r = 0; r < DEPTH; ++r)
        if (i0 + r < nt) step(ring[r], i0 + r, false);
    }
    finish_chunk(c, nt);
    // vmcnt(0): the chunk's stores are done before the next chunk's loads
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  finish_wave();
}


// Length of the combine's LDS score row (it later holds the gate input, or the
// 16 waves' partial gate sums).
static __host__ __device__ int comb_row_len(const Dims& dm) {
  const int n = dm.nsel > dm.C ? dm.nsel : dm.C;
  return ((n > 16 * 64 ? n : 16 * 64) + 3) & ~3;
}
// Per-(tile, block offset) contributions to the block scores: [nc*TPC][nb].
static __host__ __device__ int comb_contrib_len(const DecPlan& pl) { return (pl.nc * kDecTPC * pl.nb + 3) & ~3; }

// Dynamic LDS of the combine: score row, wave scales and states, top-n
// scratch, gate MLP hidden layer, tile contributions.
static size_t comb_lds_bytes(const Dims& dm, const DecPlan& pl) {
  return (size_t)comb_row_len(dm) * 4 + (size_t)pl.ns * 16 * 4 * 3 + 16 * 4 + (256 + 16 + 4) * 4 + (size_t)dm.Cg * 4 +
         (size_t)comb_contrib_len(pl) * 4;
}

// One workgroup (1024 threads) per (sequence, KV head): per-head log-sum-exp
// of the compressed branch, per-wave scales, block scores, top-n and gates.
// Global reads are laid out so that consecutive lanes read consecutive 16-byte
// pieces: the gate weights of the group's heads are contiguous per input row,
// and the per-tile score partials are read as one float4 per lane.  Loads are
// typed (T is the I/O element type) and unconditional (indices clamped, the
// result selected), so a thread's loads are all in flight together.
template <typename T>
__global__ __launch_bounds__(1024) void k_dec_combine(Dims dm, DecArgs a, DecPlan pl) {
  extern __shared__ float smem[];
  float* row = smem;                          // [nsel] block scores
  float* scl = row + comb_row_len(dm);        // [ns][16]
  float* lse2 = scl + pl.ns * 16;             // [16]
  float* mls = lse2 + 16;                     // [ns][16] wave maxima
  float* lsl = mls + pl.ns * 16;              // [ns][16] wave sums
  int* tsh = (int*)(lsl + pl.ns * 16);        // [256 + 16 + 4] top-n scratch
  float* ghid = (float*)(tsh + 256 + 16 + 4); // [Cg] gate MLP hidden layer
  float* ctb = ghid + dm.Cg;                  // [nc*TPC][nb] tile contributions
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bg = blockIdx.x, b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int G = dm.G, G3 = 3 * G;
  const DecSeq sq = dec_seq(dm, a, b);
  // linear gate: wave w takes the inputs k = k0 + w + 16 u (u < 16) and lane
  // e < 3G output e of the group (head e / 3, branch e % 3), whose weights are
  // contiguous in each input row; requested now, used at the end
  float gx[16], gw[16];
  const T* xrow = (const T*)a.x + (size_t)b * dm.C;
  const T* wcol = (const T*)a.wg + g * G3 + min(lane, G3 - 1);
  auto gate_load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int k = k0 + wave + 16 * u, kk = min(k, dm.C - 1);
      const float xv = to_f32(xrow[kk]), wv = to_f32(wcol[(size_t)kk * dm.Hq * 3]);
      gx[u] = k < dm.C ? xv : 0.f;
      gw[u] = k < dm.C && lane < G3 ? wv : 0.f;
    }
  };
  for (int i = tid; i < pl.ns * 16; i += 1024) {
    const size_t hb = (size_t)bg * pl.ns * 16 + i;
    mls[i] = a.w.part_ml[hb * 2];
    lsl[i] = a.w.part_ml[hb * 2 + 1];
  }
  if (dm.Cg == 0) gate_load(0);
  __syncthreads();
  // per-head log-sum-exp: wave h reduces head h over the waves' states
  {
    const int h = wave;
    float M = kNegInf;
    for (int c = lane; c < pl.ns; c += 64) M = fmaxf(M, mls[c * 16 + h]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float Mr = M == kNegInf ? 0.f : M;
    float L = 0.f;
    for (int c = lane; c < pl.ns; c += 64) L += lsl[c * 16 + h] * fast_exp2(mls[c * 16 + h] - Mr);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    if (lane == 0) {
      const float l2 = M == kNegInf ? kNegInf : M + __log2f(L);
      lse2[h] = l2;
      if (h < G) a.w.lse_cmp[(size_t)b * dm.Hq + g * G + h] = l2;
    }
  }
  __syncthreads();
  for (int i = tid; i < pl.ns * 16; i += 1024) {
    const float mc = mls[i], l2 = lse2[i % 16];
    const float v = (mc == kNegInf || l2 == kNegInf) ? 0.f : fast_exp2(mc - l2);
    scl[i] = v;
    a.w.cmp_scl[(size_t)bg * pl.ns * 16 + i] = v;
  }
  // block scores: sum over heads of exact probabilities remapped to blocks.
  // Tile kg's partial for block offset jj (block kg * jstep + jj) is 16
  // heads' remapped scores relative to the tile's running maxima; four lanes
  // take its four float4s, scale them to probabilities and sum over heads.
  const int ntiles = (sq.ncmp + 31) / 32;
  {
    const float4* ps4 = reinterpret_cast<const float4*>(a.w.part_ps) + (size_t)bg * pl.nc * kDecTPC * pl.nb * 4;
    const float4* tm4 = reinterpret_cast<const float4*>(a.w.part_tm) + (size_t)bg * pl.nc * kDecTPC * 4;
    const int nf = ntiles * pl.nb * 4;
    for (int f0 = 0; f0 < nf; f0 += 1024) {   // uniform trip count: the shuffles below need every lane
      const int f = f0 + tid;
      const int kg = f / (pl.nb * 4), h4 = f & 3;
      float part = 0.f;
      if (f < nf) {
        const float4 x = ps4[f], m = tm4[kg * 4 + h4];
        const float xs[4] = {x.x, x.y, x.z, x.w}, ms[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int h = h4 * 4 + e;
          const float l2 = lse2[h];
          if (h < G && ms[e] != kNegInf && l2 != kNegInf) part += xs[e] * fast_exp2(ms[e] - l2);
        }
      }
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      if (f < nf && h4 == 0) ctb[f >> 2] = part;
    }
  }
  __syncthreads();
  // each block adds the (at most a few) tiles that touch it, in tile order
  for (int j = tid; j < dm.nsel; j += 1024) {
    float val = 0.f;
    int klo = j - pl.nb + 1;
    klo = klo <= 0 ? 0 : (klo + pl.jstep - 1) / pl.jstep;
    const int khi = j < sq.nsel ? min(j / pl.jstep, ntiles - 1) : -1;
    for (int kg = klo; kg <= khi; ++kg) val += ctb[kg * pl.nb + (j - kg * pl.jstep)];
    row[j] = val;
  }
  __syncthreads();
  if (a.p_slc)
    for (int j = tid; j < dm.nsel; j += 1024) a.p_slc[(size_t)bg * dm.nsel + j] = row[j];
  int* out = a.w.idx + (size_t)bg * dm.n;
  if (dm.nsel <= 1024) {
    // rows of up to 1024 blocks: one wave, the row held in registers
    if (wave == 0) {
      const float* rows[1] = {row};
      const int ts[1] = {sq.t};
      int* outs[1] = {out};
      // inlined (a call would put the pointer arrays on a scratch stack)
      [[clang::always_inline]] wave_topn_rows<16, 1>(rows, ts, dm.ls, dm.n, outs, lane);
    }
  } else {
    __syncthreads();
    [[clang::always_inline]] block_topn<16>(row, sq.t, dm.ls, dm.n, out, tsh, tid);
  }
  // gate MLP: this sequence's hidden layer gelu(x w1 + b1) in LDS, then the
  // output layer by the waves below over it
  if (dm.Cg > 0) {
    float* gx_s = row;   // the gate input of sequence b (the score row is no longer needed)
    __syncthreads();
    for (int k = tid; k < dm.C; k += 1024) gx_s[k] = to_f32(xrow[k]);
    __syncthreads();
    for (int j = tid; j < dm.Cg; j += 1024) {
      const T* w1 = (const T*)a.gmlp.w1 + j;
      float acc = to_f32(((const T*)a.gmlp.b1)[j]);
#pragma unroll 8
      for (int k = 0; k < dm.C; ++k) acc = fmaf(gx_s[k], to_f32(w1[(size_t)k * dm.Cg]), acc);
      ghid[j] = 0.5f * acc * (1.f + erff(acc * 0.70710678118654752f));
    }
    __syncthreads();
    if (wave < G) {
      const int h = g * G + wave;
      float z[3] = {0.f, 0.f, 0.f};
      for (int k = lane; k < dm.Cg; k += 64) {
#pragma unroll
        for (int c = 0; c < 3; ++c) z[c] = fmaf(ghid[k], to_f32(((const T*)a.wg)[((size_t)k * dm.Hq + h) * 3 + c]), z[c]);
      }
#pragma unroll
      for (int c = 0; c < 3; ++c) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) z[c] += __shfl_xor(z[c], off);
      }
      if (lane < 3) {
        const float zz = (lane == 0 ? z[0] : (lane == 1 ? z[1] : z[2])) + to_f32(((const T*)a.gmlp.b2)[(size_t)h * 3 + lane]);
        a.w.gates[((size_t)b * dm.Hq + h) * 3 + lane] = 1.f / (1.f + expf(-zz));
      }
    }
    return;
  }
  // linear gate: per-wave partial sums over its inputs, then the 16 waves'
  // sums in a fixed order (the score row's space holds them)
  float z = 0.f;
  for (int k0 = 0; k0 < dm.C; k0 += 16 * 16) {
    if (k0 > 0) gate_load(k0);
#pragma unroll
    for (int u = 0; u < 16; ++u) z = fmaf(gx[u], gw[u], z);
  }
  __syncthreads();   // the top-n has read the row
  row[wave * 64 + lane] = z;
  __syncthreads();
  if (tid < G3) {
    float zz = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) zz += row[w * 64 + tid];
    a.w.gates[((size_t)b * dm.Hq + g * G + tid / 3) * 3 + tid % 3] = 1.f / (1.f + expf(-zz));
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
  // key ranges of this work item: two selected blocks or two window chunks
  // (either may be empty); one online softmax runs over both
  const DecSeq sq = dec_seq(dm, a, b);
  const bool win_item = it >= pl.nis;
  int r0[2] = {0, 0}, r1[2] = {0, 0};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!win_item) {
      const int slot = 2 * it + u;
      const int j = slot < dm.n ? a.w.idx[(size_t)bg * dm.n + slot] : -1;
      if (j >= 0) { r0[u] = j * dm.ls; r1[u] = min((j + 1) * dm.ls, sq.S); }
    } else {
      const int c = 2 * (it - pl.nis) + u;
      if (c < sq.niw) { r0[u] = sq.ws0 + c * kDecWinChunk; r1[u] = min(r0[u] + kDecWinChunk, sq.S); }
    }
  }
  const int kta = r0[0] & ~31, ktb = r0[1] & ~31;
  const int nta = r1[0] > r0[0] ? (r1[0] - kta + 31) / 32 : 0;
  const int ntile = nta + (r1[1] > r0[1] ? (r1[1] - ktb + 31) / 32 : 0);
  // first key of tile i: the first range's tiles, then the second's
  auto tkey = [&](int i) { return i < nta ? kta + 32 * i : ktb + 32 * (i - nta); };
  const float sc2 = dm.scale * kLog2e;
  const size_t kstride = (size_t)dm.Hkv * DK, vstride = (size_t)dm.Hkv * DV;
  const T* kbase = (const T*)(win_item ? a.kwcache : a.kcache) + ((size_t)b * pl.S * dm.Hkv + g) * DK;
  const T* vbase = (const T*)(win_item ? a.vwcache : a.vcache) + ((size_t)b * pl.S * dm.Hkv + g) * DV;
  const int krow = (c16 >> 2) * 8 + (c16 & 3);
  float m = kNegInf, ls = 0.f;
  f32x4 oacc[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int i) {
    const int kt = tkey(i);
    const int lo = i < nta ? r0[0] : r0[1], hi = i < nta ? r1[0] : r1[1];
    f32x4 s[2];
    Tile::scores(s, tile, qf, krow, qd);
    float v[8], mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = kt + qd * 8 + e;
      v[e] = (key >= lo && key < hi) ? s[e >> 2][e & 3] * sc2 : kNegInf;
      mx = fmaxf(mx, v[e]);
    }
    mx = fmaxf(mx, xor16f(mx, lane));
    mx = fmaxf(mx, xor32f(mx, lane));
    // lazy rescaling, as in k_dec_cmp: m is the reference of the state
    if (__builtin_amdgcn_ballot_w64(mx > m + 8.f) != 0) {
      const float mn = fmaxf(m, mx);
      const float alpha = mn == kNegInf ? 1.f : fast_exp2(m - mn);
      ls *= alpha;
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) oacc[dt] *= alpha;
      m = mn;
    }
    const float mref = m == kNegInf ? 0.f : m;
    float p[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { p[e] = fast_exp2(v[e] - mref); psum += p[e]; }
    ls += psum;
    const Frag8<T> pf = to_frag<T>(p);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) mma(oacc[dt], Tile::vfrag(tile, dt, c16, qd), pf);
  };
  // a ring of two tiles in flight (a 64-token block or aligned window chunk
  // is two tiles: the first range is requested up front, the second while
  // the first is computed)
  auto step = [&](Tile& cur, int i) {
    __syncthreads();
    cur.lstore(tile, lane);
    __syncthreads();
    if (i + 2 < ntile) cur.gload(kbase, vbase, kstride, vstride, tkey(i + 2), sq.S, lane);
    compute(i);
  };
  Tile ring[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
    if (r < ntile) ring[r].gload(kbase, vbase, kstride, vstride, tkey(r), sq.S, lane);
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
// the compressed states and of the selected/window partial states, output.
template <typename T, int DV>
__global__ __launch_bounds__(256) void k_dec_merge(Dims dm, DecArgs a, DecPlan pl) {
  extern __shared__ float sm[];
  float* swscl = sm;                  // [ni][2]
  float* cscl = swscl + pl.ni * 2;    // [ns][2]
  float* gts = cscl + pl.ns * 2;      // [2][3]
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
  for (int i = tid; i < pl.ns * 2; i += 256) cscl[i] = a.w.cmp_scl[((size_t)bg * pl.ns + i / 2) * 16 + h0 + i % 2];
  __syncthreads();
  const int hh = h0 + tid / DV, e = tid % DV;   // 2 heads x DV features (DV <= 128)
  if (tid >= 2 * DV || hh >= G) return;
  const int hl = hh - h0;
  float oc = 0.f;
#pragma unroll 8
  for (int c = 0; c < pl.ns; ++c) oc += a.w.part_o[(((size_t)bg * pl.ns + c) * 16 + hh) * DV + e] * cscl[c * 2 + hl];
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
    const size_t lds = comb_lds_bytes(dm, pl);
    if (lds > 64 * 1024)
      hipFuncSetAttribute((const void*)k_dec_combine<T>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    k_dec_combine<T><<<BG, 1024, lds, s>>>(dm, a, pl);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark()) != hipSuccess) return e;
  k_dec_sw<T, DK, DV><<<BG * pl.ni, 64, 0, s>>>(dm, a, pl);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_dec_merge<T, DV><<<BG * 8, 256, ((size_t)pl.ni * 2 + (size_t)pl.ns * 2 + 8) * sizeof(float), s>>>(dm, a, pl);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark();
}

// Whether the decode's workgroups fit a compute unit's 160 KB of LDS (the
// combine's score row and per-tile contributions grow with the cache length).
bool decode_fits(const Dims& dm) {
  const DecPlan pl = dec_plan(dm);
  const size_t merge = ((size_t)pl.ni * 2 + (size_t)pl.ns * 2 + 8) * sizeof(float);
  return comb_lds_bytes(dm, pl) <= 160 * 1024 && merge <= 160 * 1024;
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
