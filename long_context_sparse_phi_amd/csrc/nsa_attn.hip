// Selected-block attention and sliding-window attention + gated combine.
//
// Selected branch (youleyou NSA page, Top-n块选择 and 内核设计): the query of
// position t attends to the tokens <= t of its n selected blocks.  All G query
// heads of a GQA group share the block set, so one wave takes the G heads of
// one position as the 16 columns of its MFMA tiles and streams each selected
// block's keys and values through them once (group-centric loading; every
// 64-token block fetched feeds all G heads).  Online softmax across blocks.
//
// Window branch (滑动窗口): keys [t-w+1, t].  A wave owns several consecutive
// positions x G heads; the keys of its band are streamed once for all of
// them.  The epilogue reads the other two branch outputs and the gates and
// writes o = g_cmp O_cmp + g_slc O_slc + g_win O_win (最终输出计算).
//
// MFMA layout as in the compressed branch: S^T = K Q^T with keys permuted so
// lane group qd holds keys 8*qd..8*qd+7, then O^T += V^T P^T with V^T read
// from a transposed copy of V ([B, Hkv, dv, Tp]).
#include <type_traits>

#include "nsa_common.hpp"
#include "nsa_kernels.hpp"
#include "nsa_tiles.hpp"

namespace nsa {

// ---------------------------------------------------------------------------
// Fragment-ordered copies of K and V.  A selected block is gathered by one
// wave; in the natural [T, Hkv, d] layout each fragment load touches 16 key
// rows of 64 bytes, and such fragmented requests cap the load rate well below
// what contiguous requests reach.  After this re-layout every load
// instruction reads 64 lanes x 16 bytes (bf16) of contiguous memory, and one
// 32-key tile is a single contiguous run.
//
// A packed tile holds tile_ins "instructions" of 64 lanes x 8 elements.  A
// tensor [B, N, Hkv, D] contributes, per 32-key tile, either
//   key-row fragments (2*D/32): (sub, ks) -> lane (c, q) holds row
//     (c/4)*8 + c%4 + 4*sub, features ks*32 + q*8 .. +7 (A operand of K Q^T),
//   or transposed fragments (D/16): dt -> lane (c, q) holds feature
//     dt*16 + c, rows q*8 .. +7 (A operand of V^T P^T or K^T dS^T),
// starting at instruction ins0.  Rows past N are zero.
// ---------------------------------------------------------------------------
size_t frag_tiles_elems(const Dims& dm, int N, int tile_ins) {
  return (size_t)dm.B * dm.Hkv * ((N + 31) / 32) * tile_ins * 512;
}

template <typename T, int D, bool TRANS>
__global__ __launch_bounds__(256) void k_frag_pack(Dims dm, int N, const T* src, T* dst, int tile_ins, int ins0) {
  constexpr int RS = D + 8;
  constexpr int NI = TRANS ? D / 16 : 2 * D / 32;
  __shared__ __align__(16) T sr[32 * RS];
  const int nt = (N + 31) / 32;
  const int tile = blockIdx.x % nt, bg = blockIdx.x / nt;
  const int b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int k0 = tile * 32;
  for (int i = threadIdx.x; i < 32 * D / 8; i += 256) {
    const int r = i / (D / 8), c8 = i % (D / 8), key = k0 + r;
    *reinterpret_cast<Frag8<T>*>(sr + r * RS + c8 * 8) =
        key < N ? load_frag(src + ((size_t)(b * N + key) * dm.Hkv + g) * D + c8 * 8) : zero_frag<T>();
  }
  __syncthreads();
  T* out = dst + ((size_t)bg * nt + tile) * tile_ins * 512 + (size_t)ins0 * 512;
  for (int i = threadIdx.x; i < NI * 64; i += 256) {
    const int ins = i / 64, L = i % 64, c16 = L & 15, qd = L >> 4;
    Frag8<T> f;
    if constexpr (!TRANS) {
      const int sub = ins / (D / 32), ks = ins % (D / 32);
      const int r = (c16 >> 2) * 8 + (c16 & 3) + sub * 4;
      f = *reinterpret_cast<const Frag8<T>*>(sr + r * RS + ks * 32 + qd * 8);
    } else {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (float)sr[(qd * 8 + e) * RS + ins * 16 + c16];
      f = to_frag<T>(x);
    }
    *reinterpret_cast<Frag8<T>*>(out + (size_t)ins * 512 + L * 8) = f;
  }
}

template <typename T, int D>
static hipError_t frag_pack_impl(const Dims& dm, int N, const void* src, void* dst, int tile_ins, int ins0,
                                 bool trans, hipStream_t s) {
  const int grid = dm.B * dm.Hkv * ((N + 31) / 32);
  if (grid == 0) return hipSuccess;
  if (trans) k_frag_pack<T, D, true><<<grid, 256, 0, s>>>(dm, N, (const T*)src, (T*)dst, tile_ins, ins0);
  else k_frag_pack<T, D, false><<<grid, 256, 0, s>>>(dm, N, (const T*)src, (T*)dst, tile_ins, ins0);
  return hipGetLastError();
}

hipError_t launch_frag_pack(const Dims& dm, int D, int N, const void* src, void* dst, int tile_ins, int ins0,
                            bool trans, hipStream_t s) {
  const bool bf = dm.io == IO_BF16;
  switch (D) {
    case 64: return bf ? frag_pack_impl<bf16, 64>(dm, N, src, dst, tile_ins, ins0, trans, s)
                       : frag_pack_impl<float, 64>(dm, N, src, dst, tile_ins, ins0, trans, s);
    case 128: return bf ? frag_pack_impl<bf16, 128>(dm, N, src, dst, tile_ins, ins0, trans, s)
                        : frag_pack_impl<float, 128>(dm, N, src, dst, tile_ins, ins0, trans, s);
    case 192: return bf ? frag_pack_impl<bf16, 192>(dm, N, src, dst, tile_ins, ins0, trans, s)
                        : frag_pack_impl<float, 192>(dm, N, src, dst, tile_ins, ins0, trans, s);
  }
  return hipErrorInvalidValue;
}

// Selected-branch tiles: key-row K fragments, then transposed V fragments.
template <int DK, int DV> constexpr int kvf_nk() { return 2 * DK / 32; }
template <int DK, int DV> constexpr int kvf_ni() { return 2 * DK / 32 + DV / 16; }

size_t kv_frag_elems(const Dims& dm) { return frag_tiles_elems(dm, dm.T, 2 * dm.dk / 32 + dm.dv / 16); }

hipError_t launch_kv_frag(const Dims& dm, const void* k, const void* v, void* kvf, hipStream_t s) {
  const int ni = 2 * dm.dk / 32 + dm.dv / 16;
  hipError_t e = launch_frag_pack(dm, dm.dk, dm.T, k, kvf, ni, 0, false, s);
  if (e != hipSuccess) return e;
  return launch_frag_pack(dm, dm.dv, dm.T, v, kvf, ni, 2 * dm.dk / 32, true, s);
}

// One 32-key tile of a selected block, held in registers: the key fragments
// of the two MFMA sub-tiles and the V^T fragments.
template <typename T, int DK, int DV>
struct SlcTile {
  Frag8<T> k[2][DK / 32];
  Frag8<T> v[DV / 16];
};

// Walks the (block, 32-key tile) sequence of one position's selection: keys
// kt .. kt+31 of the fragment tile, of which lo <= key < kend are the block's.
struct SlcCursor {
  int si, kt, lo, kend;
};

// Register tiles in flight per wave.  bf16 tiles are small enough for a ring
// of four at one wave per SIMD (three tiles' loads in flight while one is
// computed: the gather is bound by how many bytes are outstanding); fp32 keeps
// two tiles at two waves per SIMD.
template <typename T> constexpr int slc_depth() { return sizeof(T) == 2 ? 4 : 2; }

// The selection of position t for KV head g of sequence b, walked tile by
// tile: every 32-key tile of its valid block slots goes through a ring of
// register tiles and is handed to consume(tile, cursor) in load order.
template <typename T, int DK, int DV, typename Consume>
__device__ __forceinline__ void slc_walk(const Dims& dm, const T* kvf, const int* idx, int b, int g, int t,
                                         int lane, Consume&& consume) {
  constexpr int NK = kvf_nk<DK, DV>(), NI = kvf_ni<DK, DV>();
  // the n block indices of this position, one per lane (n <= 32)
  const int* ids = idx + ((size_t)(b * dm.T + t) * dm.Hkv + g) * dm.n;
  const int myid = lane < dm.n ? ids[lane] : -1;
  const int nrow = wave_sel_row_len(myid, lane, dm.n, t, dm.ls);
  const int nt = (dm.T + 31) / 32;
  const T* kvt = kvf + (size_t)(b * dm.Hkv + g) * nt * NI * 512 + lane * 8;
  // first tile of block slot si at or after it, or si = n when none is left
  auto open_block = [&](SlcCursor& c) {
    for (; c.si < nrow; ++c.si) {
      const int j = __builtin_amdgcn_readlane(myid, c.si);
      c.lo = j * dm.ls;
      c.kt = c.lo & ~31;
      c.kend = min((j + 1) * dm.ls, t + 1);
      if (c.lo < c.kend) return;
    }
    c.si = dm.n;
  };
  auto advance = [&](SlcCursor& c) {
    c.kt += 32;
    if (c.kt < c.kend) return;
    ++c.si;
    open_block(c);
  };
  auto load_tile = [&](SlcTile<T, DK, DV>& tl, const SlcCursor& c) {
    const T* base = kvt + (size_t)(c.kt / 32) * NI * 512;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) tl.k[sub][ks] = load_frag(base + (sub * (DK / 32) + ks) * 512);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) tl.v[dt] = load_frag(base + (NK + dt) * 512);
  };
  // A ring of DEPTH register tiles, consumed in load order: after a slot's
  // tile is computed the slot is refilled with the tile DEPTH positions
  // further on, so DEPTH-1 tiles' loads are in flight during every compute.
  constexpr int DEPTH = slc_depth<T>();
  SlcTile<T, DK, DV> ring[DEPTH];
  SlcCursor rc[DEPTH];
  SlcCursor lc{0, 0, 0, 0};
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
        consume(ring[r], rc[r]);
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
}

template <typename T, int DK, int DV, typename OT>
__global__ __launch_bounds__(256, slc_depth<T>() > 2 ? 1 : 2) void k_slc(Dims dm, SlcArgs a) {
  // the wave index (hence the position t and the walk's block bounds) is
  // made visibly uniform, so the ring's control flow runs on scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  const size_t qrow = (size_t)(b * dm.T + t) * dm.Hq + hq;
  Frag8<T> qf[DK / 32];
  {
    const T* qp = (const T*)a.q + qrow * DK + qd * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qf[ks] = cv ? load_frag_nt(qp + ks * 32) : zero_frag<T>();
  }
  const float sc2 = dm.scale * kLog2e;
  float m = kNegInf, ls = 0.f;
  f32x4 oacc[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute_tile = [&](const SlcTile<T, DK, DV>& tl, const SlcCursor& c) {
    f32x4 sacc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      sacc[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) mma(sacc[sub], tl.k[sub][ks], qf[ks]);
    }
    // Scores in units of log2, masked only in tiles that cross the block's
    // range (the causal end of the current block).
    float v[8];
    if (c.kt >= c.lo && c.kt + 32 <= c.kend) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = sacc[e >> 2][e & 3] * sc2;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = c.kt + qd * 8 + e;
        v[e] = (key >= c.lo && key < c.kend) ? sacc[e >> 2][e & 3] * sc2 : kNegInf;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(v[0], v[1]), v[2]), fmaxf(fmaxf(v[3], v[4]), v[5]));
    mx = fmaxf(mx, fmaxf(v[6], v[7]));
    mx = fmaxf(mx, xor16f(mx, lane));
    mx = fmaxf(mx, xor32f(mx, lane));
    // Lazy rescaling: the reference m of a column moves only when the tile's
    // maximum exceeds it by more than 8 (so p <= 2^8); the move rescales the
    // accumulators, and is decided for the whole wave so that the common case
    // skips the multiplications.
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
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(v[e] - mref);
      psum += p[e];
    }
    ls += psum;
    const Frag8<T> pf = to_frag<T>(p);
    Frag8<T> plo;
    if constexpr (kPrecisePV<T, OT>) plo = lo_frag(p, pf);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      mma(oacc[dt], tl.v[dt], pf);
      if constexpr (kPrecisePV<T, OT>) mma(oacc[dt], tl.v[dt], plo);
    }
  };

  slc_walk<T, DK, DV>(dm, (const T*)a.kvf, a.idx, b, g, t, lane, compute_tile);
  float tot = ls + xor16f(ls, lane);
  tot += xor32f(tot, lane);
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if (cv) {
    OT* op = (OT*)a.o + qrow * DV + qd * 4;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt)
      store4_nt(op + dt * 16, oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv);
    if (qd == 0) a.lse[qrow] = (m + __log2f(tot)) * kLn2;
  }
}

template <typename T, int DK, int DV>
static hipError_t slc_impl(const Dims& dm, const SlcArgs& a, hipStream_t s) {
  dim3 grid(((dm.T + 3) / 4) * dm.B * dm.Hkv);
  if (a.o_f32) k_slc<T, DK, DV, float><<<grid, 256, 0, s>>>(dm, a);
  else k_slc<T, DK, DV, T><<<grid, 256, 0, s>>>(dm, a);
  return hipGetLastError();
}

// Calibration of the selected branch's gather: the walk of k_slc over the
// same index rows and fragment tiles, with the same launch shape, folding
// every loaded register into one word per wave instead of the attention
// arithmetic.  Its time is what the memory system takes to deliver exactly
// that access stream.
template <typename T>
__device__ __forceinline__ unsigned fold_frag(const Frag8<T>& f) {
  typedef unsigned int uv __attribute__((ext_vector_type(sizeof(Frag8<T>) / 4)));
  const uv w = __builtin_bit_cast(uv, f);
  unsigned x = 0;
#pragma unroll
  for (int e = 0; e < (int)(sizeof(Frag8<T>) / 4); ++e) x ^= w[e];
  return x;
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256, slc_depth<T>() > 2 ? 1 : 2) void k_slc_gather(Dims dm, SlcArgs a, unsigned* sink) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = (dm.T + 3) / 4;
  int unit, tile;
  xcd_map(blockIdx.x, dm.B * dm.Hkv, ntiles, unit, tile);
  const int b = unit / dm.Hkv, g = unit % dm.Hkv;
  const int t = tile * 4 + wave;
  if (t >= dm.T) return;
  unsigned acc = 0;
  slc_walk<T, DK, DV>(dm, (const T*)a.kvf, a.idx, b, g, t, lane,
                      [&](const SlcTile<T, DK, DV>& tl, const SlcCursor&) {
#pragma unroll
                        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                          for (int ks = 0; ks < DK / 32; ++ks) acc ^= fold_frag(tl.k[sub][ks]);
#pragma unroll
                        for (int dt = 0; dt < DV / 16; ++dt) acc ^= fold_frag(tl.v[dt]);
                      });
  if (lane == 0) sink[(size_t)blockIdx.x * 4 + wave] = acc;
}

template <typename T, int DK, int DV>
static hipError_t slc_gather_impl(const Dims& dm, const SlcArgs& a, unsigned* sink, hipStream_t s) {
  k_slc_gather<T, DK, DV><<<((dm.T + 3) / 4) * dm.B * dm.Hkv, 256, 0, s>>>(dm, a, sink);
  return hipGetLastError();
}

size_t slc_gather_sink_bytes(const Dims& dm) { return (size_t)((dm.T + 3) / 4) * dm.B * dm.Hkv * 4 * sizeof(unsigned); }

hipError_t launch_slc_gather(const Dims& dm, const SlcArgs& a, void* sink, hipStream_t s) {
  const bool bf = dm.io == IO_BF16;
  unsigned* u = (unsigned*)sink;
  if (dm.dk == 64 && dm.dv == 64) return bf ? slc_gather_impl<bf16, 64, 64>(dm, a, u, s) : slc_gather_impl<float, 64, 64>(dm, a, u, s);
  if (dm.dk == 128 && dm.dv == 128)
    return bf ? slc_gather_impl<bf16, 128, 128>(dm, a, u, s) : slc_gather_impl<float, 128, 128>(dm, a, u, s);
  if (dm.dk == 192 && dm.dv == 128)
    return bf ? slc_gather_impl<bf16, 192, 128>(dm, a, u, s) : slc_gather_impl<float, 192, 128>(dm, a, u, s);
  return hipErrorInvalidValue;
}

hipError_t launch_slc(const Dims& dm, const SlcArgs& a, hipStream_t s) {
  const bool bf = dm.io == IO_BF16;
  if (dm.dk == 64 && dm.dv == 64) return bf ? slc_impl<bf16, 64, 64>(dm, a, s) : slc_impl<float, 64, 64>(dm, a, s);
  if (dm.dk == 128 && dm.dv == 128) return bf ? slc_impl<bf16, 128, 128>(dm, a, s) : slc_impl<float, 128, 128>(dm, a, s);
  if (dm.dk == 192 && dm.dv == 128) return bf ? slc_impl<bf16, 192, 128>(dm, a, s) : slc_impl<float, 192, 128>(dm, a, s);
  return hipErrorInvalidValue;
}

template <typename T, int DK, int DV, int NCT, int NW, typename OT>
__global__ __launch_bounds__(NW * 64, 2) void k_win(Dims dm, WinArgs a) {
  using Tile = KVTile<T, DK, DV, true, NW * 64>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* tiles = (T*)smem_raw;                              // [2][Tile::elems]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  const int G = dm.G, PW = 16 * NCT / G, PWG = NW * PW;
  const int ntiles = (dm.T + PWG - 1) / PWG;
  int unit, tile;
  xcd_map(blockIdx.x, dm.B * dm.Hkv, ntiles, unit, tile);
  const int b = unit / dm.Hkv, g = unit % dm.Hkv;
  const int twg = tile * PWG;
  const int t0 = twg + wave * PW;
  const bool wave_live = t0 < dm.T;
  const int tl = min(dm.T - 1, t0 + PW - 1);
  Frag8<T> qf[NCT][DK / 32];
  int pos[NCT], hq[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = ct * 16 + c16;
    pos[ct] = t0 + col / G;
    hq[ct] = g * G + col % G;
    const bool v = pos[ct] < dm.T;
    const T* qp = (const T*)a.q + ((size_t)(b * dm.T + min(pos[ct], dm.T - 1)) * dm.Hq + hq[ct]) * DK + qd * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qf[ct][ks] = v ? load_frag(qp + ks * 32) : zero_frag<T>();
  }
  const float sc2 = dm.scale * kLog2e;
  float m[NCT], ls[NCT];
  f32x4 oacc[DV / 16][NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    m[ct] = kNegInf;
    ls[ct] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) oacc[dt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const size_t kstride = (size_t)dm.Hkv * DK;
  const T* kbase = (const T*)a.k + ((size_t)b * dm.T * dm.Hkv + g) * DK;
  const T* vtb = (const T*)a.vt + (size_t)(b * dm.Hkv + g) * DV * dm.Tp;
  const int krow = (c16 >> 2) * 8 + (c16 & 3);
  // keys of the workgroup's band, in 64-key tiles; each wave computes the 32-key halves of its own band
  const int kwg0 = max(0, twg - dm.w + 1) & ~63;
  const int kwg1 = min(dm.T - 1, twg + PWG - 1);
  const int nkt = (kwg1 - kwg0) / kTileKeys + 1;
  const int klo = wave_live ? (max(0, t0 - dm.w + 1) & ~31) : 0x7fffffff;
  const int khi = wave_live ? tl : -1;
  // keys in [kfull0, kfull1] are inside the window of every column of the wave
  const int kfull0 = (wave_live && t0 + PW - 1 < dm.T) ? max(0, t0 + PW - 1 - dm.w + 1) : 0x7fffffff;
  const int kfull1 = t0;

  // both MFMA blocks ask the scheduler to interleave LDS reads with MFMAs
  auto half_tile = [&](const T* tl_, int h, int kt, auto masked) {
    __builtin_amdgcn_iglp_opt(0);
    f32x4 s[2][NCT];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      Frag8<T> kf[DK / 32];
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) kf[ks] = Tile::kfrag(tl_, h * 32 + krow + sub * 4, ks, qd);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) s[sub][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) mma(s[sub][ct], kf[ks], qf[ct][ks]);
    }
    Frag8<T> pf[NCT], plo[NCT];
    float v[NCT][8], mx[NCT];
    bool grow = false;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int lo = pos[ct] - dm.w + 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[ct][e] = s[e >> 2][ct][e & 3] * sc2;
        if (masked) {
          const int key = kt + qd * 8 + e;
          v[ct][e] = (key >= lo && key <= pos[ct]) ? v[ct][e] : kNegInf;
        }
      }
      float x = fmaxf(fmaxf(fmaxf(v[ct][0], v[ct][1]), v[ct][2]), fmaxf(fmaxf(v[ct][3], v[ct][4]), v[ct][5]));
      x = fmaxf(x, fmaxf(v[ct][6], v[ct][7]));
      x = fmaxf(x, xor16f(x, lane));
      mx[ct] = fmaxf(x, xor32f(x, lane));
      grow |= mx[ct] > m[ct] + 8.f;
    }
    // Lazy rescaling: a column's reference m moves only when the half tile's
    // maximum exceeds it by more than 8 (so p <= 2^8), decided for the whole
    // wave so that the common case skips the accumulator multiplications.
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float mn = fmaxf(m[ct], mx[ct]);
        const float alpha = mn == kNegInf ? 1.f : fast_exp2(m[ct] - mn);
        ls[ct] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DV / 16; ++dt) oacc[dt][ct] *= alpha;
        m[ct] = mn;
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float mref = m[ct] == kNegInf ? 0.f : m[ct];
      float p[8], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) { p[e] = fast_exp2(v[ct][e] - mref); psum += p[e]; }
      ls[ct] += psum;
      pf[ct] = to_frag<T>(p);
      if constexpr (kPrecisePV<T, OT>) plo[ct] = lo_frag(p, pf[ct]);
    }
    __builtin_amdgcn_iglp_opt(0);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      const Frag8<T> vf = Tile::vfrag(tl_, dt * 16 + c16, h * 32, qd);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        mma(oacc[dt][ct], vf, pf[ct]);
        if constexpr (kPrecisePV<T, OT>) mma(oacc[dt][ct], vf, plo[ct]);
      }
    }
  };

  Tile ld;
  ld.gload(kbase, kstride, dm.T, vtb, dm.Tp, kwg0);
  ld.lstore(tiles);
  __syncthreads();
  for (int it = 0; it < nkt; ++it) {
    const int kt0 = kwg0 + it * kTileKeys;
    if (it + 1 < nkt) ld.gload(kbase, kstride, dm.T, vtb, dm.Tp, kt0 + kTileKeys);
    const T* tl_ = tiles + (size_t)(it & 1) * Tile::elems;
    for (int h = 0; h < 2; ++h) {
      const int kt = kt0 + h * 32;
      if (kt + 31 < klo || kt > khi) continue;
      if (kt >= kfull0 && kt + 31 <= kfull1) half_tile(tl_, h, kt, std::false_type{});
      else half_tile(tl_, h, kt, std::true_type{});
    }
    if (it + 1 < nkt) ld.lstore(tiles + (size_t)((it + 1) & 1) * Tile::elems);
    __syncthreads();
  }
  if (!wave_live) return;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    float tot = ls[ct] + xor16f(ls[ct], lane);
    tot += xor32f(tot, lane);
    if (pos[ct] >= dm.T) continue;
    const float inv = 1.f / tot;
    const size_t row = (size_t)(b * dm.T + pos[ct]) * dm.Hq + hq[ct];
    if (a.lse && qd == 0) a.lse[row] = (m[ct] + __log2f(tot)) * kLn2;
    const size_t ob = row * DV + qd * 4;
    if (a.dense) {
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt)
        store4((T*)a.o + ob + dt * 16, oacc[dt][ct][0] * inv, oacc[dt][ct][1] * inv, oacc[dt][ct][2] * inv,
               oacc[dt][ct][3] * inv);
      continue;
    }
    const float g0 = a.gates[row * 3 + 0], g1 = a.gates[row * 3 + 1], g2 = a.gates[row * 3 + 2];
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      float ow[4], oc[4], os[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ow[r] = oacc[dt][ct][r] * inv;
      if (a.o_win) store4((OT*)a.o_win + ob + dt * 16, ow[0], ow[1], ow[2], ow[3]);
      load4((const OT*)a.o_cmp + ob + dt * 16, oc);
      load4((const OT*)a.o_slc + ob + dt * 16, os);
      store4((T*)a.o + ob + dt * 16, g0 * oc[0] + g1 * os[0] + g2 * ow[0], g0 * oc[1] + g1 * os[1] + g2 * ow[1],
             g0 * oc[2] + g1 * os[2] + g2 * ow[2], g0 * oc[3] + g1 * os[3] + g2 * ow[3]);
    }
  }
}

// 8 waves x 2 column tiles per workgroup: two waves share each SIMD and the
// staged key tiles feed 16 positions x G heads.
template <typename T, int DK, int DV>
static hipError_t win_impl(const Dims& dm, const WinArgs& a, hipStream_t s) {
  constexpr int NCT = 2, NW = 8;
  const int PWG = NW * 16 * NCT / dm.G;
  const int ntiles = (dm.T + PWG - 1) / PWG;
  const size_t lds = 2 * KVTile<T, DK, DV, true, NW * 64>::elems * sizeof(T);
  auto kfn = a.o_f32 ? k_win<T, DK, DV, NCT, NW, float> : k_win<T, DK, DV, NCT, NW, T>;
  if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  kfn<<<ntiles * dm.B * dm.Hkv, NW * 64, lds, s>>>(dm, a);
  return hipGetLastError();
}

hipError_t launch_win_combine(const Dims& dm, const WinArgs& a, hipStream_t s) {
  const bool bf = dm.io == IO_BF16;
  if (dm.dk == 64 && dm.dv == 64) return bf ? win_impl<bf16, 64, 64>(dm, a, s) : win_impl<float, 64, 64>(dm, a, s);
  if (dm.dk == 128 && dm.dv == 128) return bf ? win_impl<bf16, 128, 128>(dm, a, s) : win_impl<float, 128, 128>(dm, a, s);
  if (dm.dk == 192 && dm.dv == 128) return bf ? win_impl<bf16, 192, 128>(dm, a, s) : win_impl<float, 192, 128>(dm, a, s);
  return hipErrorInvalidValue;
}

bool shapes_supported(int dk, int dv) {
  return (dk == 64 && dv == 64) || (dk == 128 && dv == 128) || (dk == 192 && dv == 128);
}

}  // namespace nsa
