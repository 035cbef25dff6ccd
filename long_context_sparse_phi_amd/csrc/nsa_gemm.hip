// Dense GEMMs of the operator and the projection layer, hand-written for
// gfx950: the gate projection, the first layer of the compression MLP phi and
// its backward, and the q/k/v/o projections.
//
//   C[m, n] (+)= sum_k A(m, k) B(k, n)
//   A(m, k) = A[m*sam + k*sak],  B(k, n) = B[k*sbk + n*sbn]
//
// Each operand is either k-contiguous (sak == 1 / sbk == 1) or contiguous
// along its other index (sam == 1 / sbn == 1), bf16 or fp32.  A workgroup of
// four waves computes a 128 x 128 tile of C with v_mfma_f32_16x16x32_bf16,
// each wave 64 x 64 (4 x 4 MFMA tiles), stepping k by 64.  Operand tiles are
// staged in LDS as 128 rows of 64 k (128-byte rows, 16-byte chunk c of row r
// stored at chunk c ^ (((r >> 1) ^ (r >> 4)) & 7): the 16 rows of a fragment
// read reach 64 distinct banks, and so do the 4-byte stores of an operand
// contiguous along m or n, which write element e ^ (g & 1) of row group g),
// double-buffered: the next tile's global
// loads are in flight in registers while the current one is multiplied.  An
// fp32 operand is staged as two bf16 planes, hi = bf16(x) and lo = bf16(x -
// hi), and enters the products as hi and lo (about 16 significant bits);
// C accumulates in fp32.  With a split of k, partial tiles go to a workspace
// and are summed in a fixed order, so results do not depend on scheduling.
#include <type_traits>

#include "nsa_common.hpp"
#include "nsa_kernels.hpp"

namespace nsa {

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kTileElems = 128 * kBK;          // one operand plane (bf16 elements)

// Value of segment s out of three, chosen by selects rather than an indexed
// read of the argument block.
template <typename V>
__device__ __forceinline__ V seg_pick(int s, V a, V b, V c) { return s == 0 ? a : (s == 1 ? b : c); }

__device__ __forceinline__ int mm_off(int r, int c) { return r * kBK + ((c ^ (((r >> 1) ^ (r >> 4)) & 7)) << 3); }

// Eight consecutive elements of an operand, as loaded (bf16 or fp32); the
// conversion to bf16 hi / lo parts waits until the LDS store, so that the
// loads stay in flight while the previous tile is multiplied.
template <typename T> struct Raw8;
template <> struct Raw8<bf16> { Frag8<bf16> v; };
template <> struct Raw8<float> { f32x4 a, b; };

template <typename T>
__device__ __forceinline__ void load8(const T* p, bool full, int nvalid, Raw8<T>& r) {
  if constexpr (sizeof(T) == 2) {
    if (full) {
      r.v = load_frag(p);
    } else {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = e < nvalid ? (float)p[e] : 0.f;
      r.v = to_frag_bf16(x);
    }
  } else {
    if (full) {
      r.a = *reinterpret_cast<const f32x4*>(p);
      r.b = *reinterpret_cast<const f32x4*>(p + 4);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r.a[e] = e < nvalid ? p[e] : 0.f;
        r.b[e] = e + 4 < nvalid ? p[e + 4] : 0.f;
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ void split8(const Raw8<T>& r, Frag8<bf16>& hi, Frag8<bf16>& lo) {
  if constexpr (sizeof(T) == 2) {
    hi = r.v;
  } else {
    const float x[8] = {r.a[0], r.a[1], r.a[2], r.a[3], r.b[0], r.b[1], r.b[2], r.b[3]};
    split_bf16(x, hi, lo);
  }
}

// One operand of a 128-row x 64-k tile: rows r0 .. r0+127 (of nrows), k from
// k0 (of K).  KC: element (r, k) at X[r*srow + k]; otherwise at X[r + k*sk].
template <typename T, bool KC>
struct Stage {
  static constexpr bool SPLIT = sizeof(T) == 4;
  static constexpr int NT = KC ? 4 : 2;        // loads per thread
  Raw8<T> raw[NT][KC ? 1 : 2];

  __device__ __forceinline__ void load(const T* X, long long stride, int r0, int nrows, int k0, int K, int tid) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int idx = tid + 256 * i;
      if constexpr (KC) {
        // chunk of 8 k of one row
        const int r = idx >> 3, c = idx & 7;
        const int rg = r0 + r, kg = k0 + c * 8;
        const bool live = rg < nrows && kg < K;
        const T* p = X + (long long)(live ? rg : 0) * stride + (live ? kg : 0);
        load8<T>(p, live && kg + 8 <= K, live ? K - kg : 0, raw[i][0]);
      } else {
        // 8 consecutive rows at k and k + 1
        const int kp = idx >> 4, rgp = idx & 15;
        const int rg = r0 + rgp * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kg = k0 + 2 * kp + h;
          const bool live = kg < K && rg < nrows;
          const T* p = X + (live ? (long long)kg * stride + rg : 0);
          load8<T>(p, live && rg + 8 <= nrows, live ? nrows - rg : 0, raw[i][h]);
        }
      }
    }
  }

  __device__ __forceinline__ void store(bf16* phi, bf16* plo, int tid) const {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int idx = tid + 256 * i;
      if constexpr (KC) {
        const int r = idx >> 3, c = idx & 7;
        Frag8<bf16> hi, lo;
        split8<T>(raw[i][0], hi, lo);
        *reinterpret_cast<Frag8<bf16>*>(phi + mm_off(r, c)) = hi;
        if constexpr (SPLIT) *reinterpret_cast<Frag8<bf16>*>(plo + mm_off(r, c)) = lo;
      } else {
        const int kp = idx >> 4, rgp = idx & 15;
        const int k = 2 * kp;
        Frag8<bf16> hi[2], lo[2];
        split8<T>(raw[i][0], hi[0], lo[0]);
        split8<T>(raw[i][1], hi[1], lo[1]);
        // store e writes row rgp*8 + (e ^ odd): rows of both parities in every
        // store instruction, which with the swizzle spreads it over all banks
        const bool odd = rgp & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = rgp * 8 + (e ^ (int)odd);
          const int o = mm_off(r, k >> 3) + (k & 7);
          bf16x2v v;
          v[0] = odd ? hi[0].v[e ^ 1] : hi[0].v[e];
          v[1] = odd ? hi[1].v[e ^ 1] : hi[1].v[e];
          *reinterpret_cast<bf16x2v*>(phi + o) = v;
          if constexpr (SPLIT) {
            bf16x2v w;
            w[0] = odd ? lo[0].v[e ^ 1] : lo[0].v[e];
            w[1] = odd ? lo[1].v[e ^ 1] : lo[1].v[e];
            *reinterpret_cast<bf16x2v*>(plo + o) = w;
          }
        }
      }
    }
  }
};

// blockIdx.z = batch * nsplit + split.  Two register sets of staged tiles:
// while tile i is multiplied from LDS, tile i+1 (loaded one step earlier)
// waits in one set and tile i+2's loads are in flight into the other.
template <typename TA, typename TB, bool AKC, bool BKC>
__global__ __launch_bounds__(256) void k_mm(MmArgs g, int kc, int nsplit, float* part) {
  constexpr bool SA = sizeof(TA) == 4, SB = sizeof(TB) == 4;
  constexpr int PA = SA ? 2 : 1, PB = SB ? 2 : 1;
  constexpr int BUF = (PA + PB) * kTileElems;        // one pipeline stage
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16* lds = (bf16*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  // Persistent: the workgroups of a (batch, split) plane walk its output
  // tiles with a stride of the grid width, which is a multiple of 8 when
  // the grid is smaller than the tile count (so tile lid keeps XCD lid % 8).
  // segments: n segments pick B and C per column tile, k segments pick A
  // and B per k step (seg_pick keeps the choice in scalar registers)
  const bool nsegs = g.nseg > 1 && !g.seg_k, ksegs = g.nseg > 1 && g.seg_k;
  const int soff[3] = {g.seg[0].off, g.seg[1].off, g.seg[2].off};
  const int ncol = nsegs ? seg_tiles(g.nseg, soff, g.N, kBN) : (g.N + kBN - 1) / kBN;
  const int nrow = (g.M + kBM - 1) / kBM;
  for (int lid = blockIdx.x; lid < ncol * nrow; lid += gridDim.x) {
    int mt, nt;
    gemm_tile_order(lid, ncol, nrow, mt, nt);
    int sn = 0, n0 = nt * kBN, Nl = g.N;     // segment, first column in it, its width
    if (nsegs) {
      seg_tile(nt, g.nseg, soff, g.N, kBN, sn, n0);
      Nl = seg_width(sn, g.nseg, soff, g.N);
    }
    const int m0 = mt * kBM;
    const int split = blockIdx.z % nsplit, bat = blockIdx.z / nsplit;
    const int kbeg = split * kc, kend = min(g.K, kbeg + kc);
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const TA* A = (const TA*)g.A + bat * g.bsa;
    const TB* B = nsegs ? (const TB*)seg_pick(sn, g.seg[0].B, g.seg[1].B, g.seg[2].B) : (const TB*)g.B + bat * g.bsb;
    // A rows are m (stride sam) and B rows are n (stride sbn); k-contiguous
    // operands step rows by their row stride, the others step k by theirs
    const long long as = AKC ? g.sam : g.sak;
    const long long bs = nsegs ? (BKC ? seg_pick(sn, g.seg[0].sbn, g.seg[1].sbn, g.seg[2].sbn)
                                      : seg_pick(sn, g.seg[0].sbk, g.seg[1].sbk, g.seg[2].sbk))
                               : (BKC ? g.sbn : g.sbk);
    Stage<TA, AKC> sa[2];
    Stage<TB, BKC> sb[2];
    f32x4 acc[4][4];
  #pragma unroll
    for (int i = 0; i < 4; ++i)
  #pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;
    auto gload = [&](auto set, int t) {
      constexpr int S = decltype(set)::value;
      int k0 = kbeg + t * kBK, kl = kend;
      const TA* Ap = A;
      const TB* Bp = B;
      long long ap = as, bp = bs;
      if (ksegs) {
        // the k segment holding this step, and k relative to its start
        const int sk = (g.nseg > 2 && k0 >= soff[2]) ? 2 : (k0 >= soff[1] ? 1 : 0);
        const int ko = seg_pick(sk, soff[0], soff[1], soff[2]);
        kl = min(kend, ko + seg_width(sk, g.nseg, soff, g.K)) - ko;
        k0 -= ko;
        Ap = (const TA*)seg_pick(sk, g.seg[0].A, g.seg[1].A, g.seg[2].A);
        Bp = (const TB*)seg_pick(sk, g.seg[0].B, g.seg[1].B, g.seg[2].B);
        ap = AKC ? seg_pick(sk, g.seg[0].sam, g.seg[1].sam, g.seg[2].sam)
                 : seg_pick(sk, g.seg[0].sak, g.seg[1].sak, g.seg[2].sak);
        bp = BKC ? seg_pick(sk, g.seg[0].sbn, g.seg[1].sbn, g.seg[2].sbn)
                 : seg_pick(sk, g.seg[0].sbk, g.seg[1].sbk, g.seg[2].sbk);
      }
      sa[S].load(Ap, ap, m0, g.M, k0, kl, tid);
      sb[S].load(Bp, bp, n0, Nl, k0, kl, tid);
    };
    auto lstore = [&](auto set) {
      constexpr int S = decltype(set)::value;
      bf16* base = lds + (size_t)S * BUF;
      sa[S].store(base, base + kTileElems, tid);
      sb[S].store(base + PA * kTileElems, base + (PA + 1) * kTileElems, tid);
    };
    auto compute = [&](auto set) {
      constexpr int S = decltype(set)::value;
      const bf16* base = lds + (size_t)S * BUF;
      const bf16* ah = base;
      const bf16* al = base + kTileElems;
      const bf16* bh = base + PA * kTileElems;
      const bf16* bl = bh + kTileElems;
  #pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        Frag8<bf16> af[4], bfr[4], alo[SA ? 4 : 1], blo[SB ? 4 : 1];
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int o = mm_off(wm + i * 16 + c16, kk * 4 + qd);
          af[i] = *reinterpret_cast<const Frag8<bf16>*>(ah + o);
          if constexpr (SA) alo[i] = *reinterpret_cast<const Frag8<bf16>*>(al + o);
        }
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int o = mm_off(wn + j * 16 + c16, kk * 4 + qd);
          bfr[j] = *reinterpret_cast<const Frag8<bf16>*>(bh + o);
          if constexpr (SB) blo[j] = *reinterpret_cast<const Frag8<bf16>*>(bl + o);
        }
  #pragma unroll
        for (int i = 0; i < 4; ++i)
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            mma(acc[i][j], af[i], bfr[j]);
            if constexpr (SA) mma(acc[i][j], alo[i], bfr[j]);
            if constexpr (SB) mma(acc[i][j], af[i], blo[j]);
          }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // step t: set S holds nothing pending (its tile t is in LDS buffer S), the
    // other set holds tile t+1; tile t+2 is requested into set S
    auto step = [&](auto set, int t) {
      constexpr int S = decltype(set)::value;
      using O = std::integral_constant<int, 1 - S>;
      if (t + 2 < nk) gload(set, t + 2);
      compute(set);
      if (t + 1 < nk) lstore(O{});
      __syncthreads();
    };
    if (nk > 0) gload(I0{}, 0);
    if (nk > 1) gload(I1{}, 1);
    if (nk > 0) lstore(I0{});
    __syncthreads();
    for (int t = 0; t < nk; t += 2) {
      step(I0{}, t);
      if (t + 1 < nk) step(I1{}, t + 1);
    }
    // C tile (or this split's partial tile) through LDS: each wave writes its
    // 64 x 64 fp32 tile (row stride 68 floats: the four row groups of a write
    // land on distinct banks), then stores it row by row, four consecutive
    // values per lane.  The k loop's last barrier has freed the LDS.
    float* ep = (float*)smem_raw + (size_t)wave * 64 * 68;
  #pragma unroll
    for (int i = 0; i < 4; ++i)
  #pragma unroll
      for (int j = 0; j < 4; ++j)
  #pragma unroll
        for (int r = 0; r < 4; ++r) ep[(i * 16 + qd * 4 + r) * 68 + j * 16 + c16] = acc[i][j][r];
    __syncthreads();
    const bool to_part = part != nullptr;
    float* pz = to_part ? part + (size_t)blockIdx.z * g.M * g.N : nullptr;
    // an n segment's columns go to its own C, or at their place in the
    // full-width partial rows
    void* Cs = nsegs ? seg_pick(sn, g.seg[0].C, g.seg[1].C, g.seg[2].C) : g.C;
    const long long ldc = nsegs ? seg_pick(sn, g.seg[0].ldc, g.seg[1].ldc, g.seg[2].ldc) : g.ldc;
    const int pcol = to_part && nsegs ? seg_pick(sn, soff[0], soff[1], soff[2]) : 0;
    const long long ld = to_part ? g.N : ldc;
    const long long cb = to_part ? 0 : bat * g.bsc;
    const bool c16b = !to_part && g.c_bf16;
    const bool acc_c = !to_part && g.accumulate;
    const uintptr_t cbase = to_part ? (uintptr_t)(pz + pcol) : (uintptr_t)Cs + (uintptr_t)cb * (c16b ? 2 : 4);
    // four-value vectors need 16-byte (fp32) or 8-byte (bf16) aligned rows
    const bool vec = ld % 4 == 0 && cbase % (c16b ? 8 : 16) == 0;
    const int col = (lane & 15) * 4;
    const int n = n0 + wn + col;
  #pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int row = it * 4 + (lane >> 4);
      const int m = m0 + wm + row;
      if (m >= g.M || n >= Nl) continue;
      const f32x4 v = *reinterpret_cast<const f32x4*>(ep + row * 68 + col);
      const long long o = (long long)m * ld + pcol + n;
      if (c16b) {
        bf16* cp = (bf16*)Cs + cb + o;
        if (vec && n + 4 <= Nl) {
          store_col4(cp, (bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]);
        } else {
          for (int e = 0; e < 4 && n + e < Nl; ++e) cp[e] = (bf16)v[e];
        }
      } else {
        float* cp = to_part ? pz + o : (float*)Cs + cb + o;
        if (vec && n + 4 <= Nl) {
          f32x4 w = v;
          if (acc_c) {
            const f32x4 old = *reinterpret_cast<const f32x4*>(cp);
            w = f32x4{old[0] + v[0], old[1] + v[1], old[2] + v[2], old[3] + v[3]};
          }
          *reinterpret_cast<f32x4*>(cp) = w;
        } else {
          for (int e = 0; e < 4 && n + e < Nl; ++e) cp[e] = acc_c ? cp[e] + v[e] : v[e];
        }
      }
    }
    // the epilogue's LDS reads are done before the next tile is staged
    __syncthreads();
  }
}

// Sums the split partials of each batch in split order into C.
__global__ __launch_bounds__(256) void k_mm_reduce(MmArgs g, int nsplit, const float* __restrict__ part) {
  const size_t mn = (size_t)g.M * g.N;
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int bat = blockIdx.y;
  if (id >= mn) return;
  const int m = (int)(id / g.N), n = (int)(id % g.N);
  float s = 0.f;
  for (int z = 0; z < nsplit; ++z) s += part[((size_t)bat * nsplit + z) * mn + id];
  // n segments: the column's segment and its place in that segment's C
  int sn = 0;
  if (g.nseg > 1 && !g.seg_k) sn = (g.nseg > 2 && n >= g.seg[2].off) ? 2 : (n >= g.seg[1].off ? 1 : 0);
  const bool segs = g.nseg > 1 && !g.seg_k;
  void* C = segs ? seg_pick(sn, g.seg[0].C, g.seg[1].C, g.seg[2].C) : g.C;
  const long long ldc = segs ? seg_pick(sn, g.seg[0].ldc, g.seg[1].ldc, g.seg[2].ldc) : g.ldc;
  const int nl = segs ? n - seg_pick(sn, g.seg[0].off, g.seg[1].off, g.seg[2].off) : n;
  const long long o = bat * g.bsc + (long long)m * ldc + nl;
  if (g.c_bf16) {
    ((bf16*)C)[o] = (bf16)s;
  } else {
    float* cp = (float*)C + o;
    *cp = g.accumulate ? *cp + s : s;
  }
}

template <typename TA, typename TB, bool AKC, bool BKC>
hipError_t mm_launch(const MmArgs& g, int nsplit, int kc, float* part, hipStream_t s) {
  constexpr int PA = sizeof(TA) == 4 ? 2 : 1, PB = sizeof(TB) == 4 ? 2 : 1;
  // the operand pipeline, or the epilogue's four 64 x 68 fp32 wave tiles
  const size_t pipe = 2 * (size_t)(PA + PB) * kTileElems * sizeof(bf16), epi = (size_t)4 * 64 * 68 * sizeof(float);
  const size_t lds = pipe > epi ? pipe : epi;
  auto kfn = k_mm<TA, TB, AKC, BKC>;
  if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  // two workgroups per CU over all planes; below the tile count the width is
  // rounded down to a multiple of 8 (the XCD count)
  int soff[3] = {g.seg[0].off, g.seg[1].off, g.seg[2].off};
  const int ncol = g.nseg > 1 && !g.seg_k ? seg_tiles(g.nseg, soff, g.N, kBN) : (g.N + kBN - 1) / kBN;
  const int ntile = ncol * ((g.M + kBM - 1) / kBM), planes = nsplit * g.batch;
  const int cap = 512 / planes > 8 ? (512 / planes) & ~7 : 8;
  dim3 grid(ntile > cap ? cap : ntile, 1, planes);
  kfn<<<grid, 256, lds, s>>>(g, kc, nsplit, nsplit > 1 ? part : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  const size_t mn = (size_t)g.M * g.N;
  k_mm_reduce<<<dim3((unsigned)((mn + 255) / 256), g.batch), 256, 0, s>>>(g, nsplit, part);
  return hipGetLastError();
}

template <typename TA, typename TB>
hipError_t mm_layout(const MmArgs& g, bool akc, bool bkc, int nsplit, int kc, float* part, hipStream_t s) {
  if (akc) return bkc ? mm_launch<TA, TB, true, true>(g, nsplit, kc, part, s)
                      : mm_launch<TA, TB, true, false>(g, nsplit, kc, part, s);
  return bkc ? mm_launch<TA, TB, false, true>(g, nsplit, kc, part, s)
             : mm_launch<TA, TB, false, false>(g, nsplit, kc, part, s);
}

bool aligned_elems(const void* p, long long stride, int esz) {
  return ((uintptr_t)p & 15) == 0 && (stride * esz) % 16 == 0;
}


// ---------------------------------------------------------------------------
// Exact fp32 path: operands staged in LDS as fp32, 16x16x4 fp32 MFMAs.
// ---------------------------------------------------------------------------

// blockIdx.z = split index: k range [z*kc, (z+1)*kc); with a split the result
// goes to part[z][M][N] and is summed afterwards in split order.
template <typename TA, typename TB>
__global__ __launch_bounds__(256) void k_gemm(Gemm gm, int kc, float* part) {
  __shared__ float As[32][64 + 4];
  __shared__ float Bs[32][64 + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kq = lane >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int kbeg = blockIdx.z * kc, kend = min(gm.K, kbeg + kc);
  const TA* A = (const TA*)gm.A;
  const TB* B = (const TB*)gm.B;
  f32x4 acc[2][2];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool a_k_fast = gm.sak == 1, b_n_fast = gm.sbn == 1;
  for (int k0 = kbeg; k0 < kend; k0 += 32) {
    for (int i = tid; i < 64 * 32; i += 256) {
      int mm, kk;
      if (a_k_fast) { kk = i & 31; mm = i >> 5; } else { mm = i & 63; kk = i >> 6; }
      const int m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < gm.M && k < kend) ? to_f32(A[m * gm.sam + k * gm.sak]) : 0.f;
      int nn, kb;
      if (b_n_fast) { nn = i & 63; kb = i >> 6; } else { kb = i & 31; nn = i >> 5; }
      const int n = n0 + nn, k2 = k0 + kb;
      Bs[kb][nn] = (n < gm.N && k2 < kend) ? to_f32(B[k2 * gm.sbk + n * gm.sbn]) : 0.f;
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
        if (part) {
          part[((size_t)blockIdx.z * gm.M + m) * gm.N + n] = acc[i][j][r];
        } else {
          float* cp = gm.C + (long long)m * gm.ldc + n;
          *cp = gm.accumulate ? *cp + acc[i][j][r] : acc[i][j][r];
        }
      }
    }
}

__global__ __launch_bounds__(256) void k_gemm_reduce(Gemm gm, int nsplit, const float* __restrict__ part) {
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (size_t)gm.M * gm.N) return;
  const int m = id / gm.N, n = id % gm.N;
  float s = 0.f;
  for (int z = 0; z < nsplit; ++z) s += part[(size_t)z * gm.M * gm.N + id];
  float* cp = gm.C + (long long)m * gm.ldc + n;
  *cp = gm.accumulate ? *cp + s : s;
}

// Splits K so that about 512 workgroups run; partials need nsplit*M*N floats of part.
template <typename TA, typename TB>
hipError_t gemm_t(const Gemm& g, float* part, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int tiles = ((g.N + 63) / 64) * ((g.M + 63) / 64);
  int nsplit = part ? (512 + tiles - 1) / tiles : 1;
  nsplit = min(nsplit, min(kGemmMaxSplit, max(1, g.K / 256)));
  const int kc = ((g.K + nsplit - 1) / nsplit + 31) & ~31;
  nsplit = (g.K + kc - 1) / kc;
  dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, nsplit);
  if (nsplit == 1) {
    k_gemm<TA, TB><<<grid, 256, 0, s>>>(g, kc, nullptr);
    return hipGetLastError();
  }
  k_gemm<TA, TB><<<grid, 256, 0, s>>>(g, kc, part);
  const size_t mn = (size_t)g.M * g.N;
  k_gemm_reduce<<<(unsigned)((mn + 255) / 256), 256, 0, s>>>(g, nsplit, part);
  return hipGetLastError();
}


}  // namespace

hipError_t gemm_exact(const Gemm& g, bool a_f32, bool b_f32, float* part, hipStream_t s) {
  if (!a_f32) return b_f32 ? gemm_t<bf16, float>(g, part, s) : gemm_t<bf16, bf16>(g, part, s);
  return b_f32 ? gemm_t<float, float>(g, part, s) : gemm_t<float, bf16>(g, part, s);
}

int mm_split(const MmArgs& g, int max_split) {
  const long long tiles = (long long)((g.N + kBN - 1) / kBN) * ((g.M + kBM - 1) / kBM) * g.batch;
  int ns = (int)((512 + tiles - 1) / tiles);
  ns = min(ns, min(max_split, max(1, g.K / 512)));
  return max(ns, 1);
}

bool mm_supported(const MmArgs& g, bool a_f32, bool b_f32) {
  const int ea = a_f32 ? 4 : 2, eb = b_f32 ? 4 : 2;
  const bool akc = g.sak == 1, bkc = g.sbk == 1;
  if (!akc && g.sam != 1) return false;
  if (!bkc && g.sbn != 1) return false;
  if (g.nseg <= 1) return aligned_elems(g.A, akc ? g.sam : g.sak, ea) && aligned_elems(g.B, bkc ? g.sbn : g.sbk, eb);
  // segments: batch 1, increasing offsets from 0, every segment's operands in
  // the top-level layout, k segments in whole 64-wide k steps
  if (g.nseg > 3 || g.batch != 1 || g.seg[0].off != 0) return false;
  const int ext = g.seg_k ? g.K : g.N;
  for (int s = 0; s < g.nseg; ++s) {
    const MmSeg& q = g.seg[s];
    const int end = s + 1 < g.nseg ? g.seg[s + 1].off : ext;
    if (end <= q.off) return false;
    if (g.seg_k && s + 1 < g.nseg && (end - q.off) % kBK != 0) return false;
    if ((q.sbk == 1) != bkc || (!bkc && q.sbn != 1)) return false;
    if (!aligned_elems(q.B, bkc ? q.sbn : q.sbk, eb)) return false;
    if (g.seg_k) {
      if ((q.sak == 1) != akc || (!akc && q.sam != 1)) return false;
      if (!aligned_elems(q.A, akc ? q.sam : q.sak, ea)) return false;
    }
  }
  return g.seg_k || aligned_elems(g.A, akc ? g.sam : g.sak, ea);
}

hipError_t mm(const MmArgs& g, bool a_f32, bool b_f32, int nsplit, float* part, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (!mm_supported(g, a_f32, b_f32) || (g.c_bf16 && g.accumulate)) return hipErrorInvalidValue;
  nsplit = max(1, nsplit);
  if (nsplit > 1 && !part) return hipErrorInvalidValue;
  const int kc = ((g.K + nsplit - 1) / nsplit + kBK - 1) / kBK * kBK;
  nsplit = g.K > 0 ? (g.K + kc - 1) / kc : 1;
  const bool akc = g.sak == 1, bkc = g.sbk == 1;
  if (!a_f32) return b_f32 ? mm_layout<bf16, float>(g, akc, bkc, nsplit, kc, part, s)
                           : mm_layout<bf16, bf16>(g, akc, bkc, nsplit, kc, part, s);
  return b_f32 ? mm_layout<float, float>(g, akc, bkc, nsplit, kc, part, s)
               : mm_layout<float, bf16>(g, akc, bkc, nsplit, kc, part, s);
}

}  // namespace nsa
