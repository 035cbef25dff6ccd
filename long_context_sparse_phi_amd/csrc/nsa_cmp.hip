// Compressed-attention branch, importance scores and top-n block selection.
//
// youleyou NSA page, 重要性分数计算 / Top-n块选择: the compressed branch's softmax
// probabilities p_cmp[t,h,i] are reused as importance scores.  They are remapped
// from compression blocks (l tokens every d) to selection blocks (l' tokens):
// selection block j receives from compression block i the overlap of their
// token ranges in units of d; the result is summed over the G query heads of
// the GQA group and the n top blocks are kept, block 0 and the two blocks
// holding t and the one before always among them, lower index winning a tie.
//
// Because the scores are normalised per head before the head sum, the
// normaliser of every (t, h) must be known first: pass A computes the
// log-sum-exp over the visible compressed keys; pass B recomputes the scores,
// forms exact probabilities, accumulates O_cmp = P V_cmp, remaps P onto
// selection blocks with one more MFMA (P times the constant 0/1/2 overlap
// matrix; for bf16 inputs P enters it as a bf16 hi + lo pair, about 16
// significant bits with fp32's exponent range, so a block 80 nats below the
// row maximum still ranks by its own value), sums over heads with cross-lane
// adds, keeps each position's score row in LDS and runs the top-n selection
// there.
//
// Layout of the work: a wave owns 16*NCT query columns = (positions x G heads
// of one KV group); MFMA tiles compute S^T = K Q^T (16 keys x 16 columns) so
// that every lane holds one column's scores for 8 keys, which is directly the
// B operand of O^T = V^T P^T.  Keys inside a 32-key tile are permuted so that
// lane group qd (= lane/16) ends up holding keys 8*qd .. 8*qd+7.
#include <type_traits>

#include "nsa_common.hpp"
#include "nsa_kernels.hpp"
#include "nsa_tiles.hpp"

namespace nsa {

// ---------------------------------------------------------------------------
// One kernel for both passes.  A workgroup of NW waves owns PWG consecutive
// positions of one (batch, KV head); all waves need the same compressed keys,
// so KT-key tiles of K_cmp (and, in pass B, of V_cmp^T) are staged once in LDS
// per workgroup, double-buffered: the next tile's global loads are in flight
// (in registers) while the current tile is computed from LDS.
// ---------------------------------------------------------------------------
// LDS row stride of the padded (fp32) V^T tile (elements)
template <int KT>
constexpr int cmp_vs() { return KT + 8; }

// V^T tile layout.  fp32: rows of KT keys padded to KT + 8.  bf16: rows of
// 128 bytes (8 chunks of 8 keys) without padding, chunk c of row R stored at
// c ^ ((R >> 1) & 7); with 32-key tiles a 128-byte row holds dv rows R and
// R + DV/2 (chunks 0-3 and 4-7).  Measured on gfx950, both the 16-lane
// fragment reads (16 consecutive rows, one chunk column) and the stores
// (8 lanes per row) of this layout are free of bank conflicts, while padded
// 32- and 64-key rows are not.
template <typename T, int KT>
struct VtLayout {
  static constexpr bool kSwz = sizeof(T) == 2;
  static constexpr int CPR = KT / 8;                  // chunks per dv row
  template <int DV>
  static constexpr int rows() { return kSwz ? DV * CPR / 8 : DV; }
  // element offset of chunk c (8 keys) of dv row r
  template <int DV>
  __device__ static int off(int r, int c) {
    if constexpr (kSwz) {
      constexpr int NR = rows<DV>();
      const int R = r % NR, cc = (r / NR) * CPR + c;
      return R * 64 + ((cc ^ ((R >> 1) & 7)) << 3);
    } else {
      return r * cmp_vs<KT>() + c * 8;
    }
  }
  template <int DV>
  static constexpr size_t elems() { return kSwz ? (size_t)DV * KT : (size_t)DV * cmp_vs<KT>(); }
};

// K tile rows are unpadded with XOR-swizzled 16-byte chunks (kchunk_off).
template <typename T, int DK, int DV, bool PB, int KT>
constexpr size_t cmp_tile_elems() {
  return (size_t)KT * DK + (PB ? VtLayout<T, KT>::template elems<DV>() : 0);
}

// GS, NJ: group size and number of 16-block remap column tiles fixed at
// compile time (0: read from the arguments).
template <typename T, int DK, int DV, int NCT, int NW, bool PB, typename OT, int GS, int NJ, int KT>
__global__ __launch_bounds__(NW * 64, 2) void k_cmp(Dims dm, CmpArgs a, int nselp, int njt_arg) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  constexpr size_t TE = cmp_tile_elems<T, DK, DV, PB, KT>();
  using VL = VtLayout<T, KT>;
  constexpr int NH = KT / 32;                               // 32-key halves per tile
  constexpr int NT = NW * 64;
  T* tiles = (T*)smem_raw;                                  // [2][TE]
  // With bf16 tiles, the group size fixed at compile time and four waves,
  // the wave index is read through readfirstlane so that the compiler knows
  // it is uniform: everything derived from it (positions, loop bounds, tile
  // addresses, LDS destinations) then lives in scalar registers.  The other
  // instances keep the per-lane form, which is what fits their register
  // budget.
  constexpr bool kScalarWave = GS != 0 && NW == 4 && sizeof(T) == 2;
  const int lane = threadIdx.x & 63;
  const int wave = kScalarWave ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  const int G = GS ? GS : dm.G, PW = 16 * NCT / G, PWG = NW * PW;
  const int njt = NJ ? NJ : njt_arg;
  const int ntiles = (dm.T + PWG - 1) / PWG;
  int unit, tile;
  xcd_map(blockIdx.x, dm.B * dm.Hkv, ntiles, unit, tile);
  const int b = unit / dm.Hkv, g = unit % dm.Hkv;
  const int twg = tile * PWG;
  const int t0 = twg + wave * PW;
  const bool wave_live = t0 < dm.T;
  const int nmax_wg = ncmp_visible(min(dm.T - 1, twg + PWG - 1), dm.l, dm.d);
  const int nmax = wave_live ? ncmp_visible(min(dm.T - 1, t0 + PW - 1), dm.l, dm.d) : 0;
  // keys below nfull are visible to every column of the wave (no masking)
  const int nfull = (wave_live && t0 + PW - 1 < dm.T) ? ncmp_visible(t0, dm.l, dm.d) : 0;
  float* prow = (float*)(smem_raw + 2 * TE * sizeof(T)) + (size_t)wave * PW * nselp;
  if (PB)
    for (int i = lane; i < PW * nselp; i += 64) prow[i] = 0.f;

  const T* q = (const T*)a.q;
  Frag8<T> qf[NCT][DK / 32];
  int pos[NCT], hq[NCT], nvis[NCT];
  float lse2[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = ct * 16 + c16;
    pos[ct] = t0 + col / G;
    hq[ct] = g * G + col % G;
    const bool v = pos[ct] < dm.T;
    nvis[ct] = v ? ncmp_visible(pos[ct], dm.l, dm.d) : 0;
    const size_t row = (size_t)(b * dm.T + min(pos[ct], dm.T - 1)) * dm.Hq + hq[ct];
    lse2[ct] = (PB && v && nvis[ct] > 0) ? a.lse[row] * kLog2e : 0.f;
    const T* qp = q + row * DK + qd * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qf[ct][ks] = v ? load_frag(qp + ks * 32) : zero_frag<T>();
  }
  // remap weights (small integers, exact in bf16); bf16 inputs remap P as a
  // hi + lo pair
  constexpr bool kSplitRemap = sizeof(T) == 2;
  Frag8<T> wf[2];
  if (PB) {
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      float w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = jt < njt ? remap_weight(qd * 8 + e, jt * 16 + c16, dm.l, dm.d, dm.ls) : 0.f;
      wf[jt] = to_frag<T>(w);
    }
  }
  const float sc2 = dm.scale * kLog2e;
  float m[NCT], mr[NCT], ls[NCT];
  f32x4 oacc[PB ? DV / 16 : 1][NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    m[ct] = kNegInf;
    mr[ct] = kNegInf;
    ls[ct] = 0.f;
#pragma unroll
    for (int dt = 0; dt < (PB ? DV / 16 : 1); ++dt) oacc[dt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // cooperative tile loader
  constexpr int KCH = KT * DK / 8 / NT;            // 16-byte chunks per thread (K)
  constexpr int VCH = PB ? DV * KT / 8 / NT : 0;
  static_assert(KCH * NT == KT * DK / 8, "K tile must split evenly over the workgroup");
  static_assert(!PB || VCH * NT == DV * KT / 8, "V tile must split evenly over the workgroup");
  Frag8<T> kr[KCH], vr[VCH > 0 ? VCH : 1];
  const T* kcb = (const T*)a.kc + ((size_t)b * dm.ncmp * dm.Hkv + g) * DK;
  const T* vtb = (const T*)a.vct + (size_t)(b * dm.Hkv + g) * DV * dm.ncmp_pad;
  // bf16 tiles go from global memory straight into LDS (one 16-byte chunk
  // per lane and load, lane i of a load writing chunk i of a 1 KB window), so
  // each thread loads the chunk that belongs at its LDS position under the
  // swizzled layouts; fp32 tiles pass through registers.
  constexpr bool kDMA = sizeof(T) == 2;
  // per-thread chunk offsets, the same for every tile: global (elements from
  // the tile's first key) and LDS
  const int kstride = dm.Hkv * DK;
  int kgo[KCH], klo[KCH], krw[KCH], vgo[VCH > 0 ? VCH : 1], vlo[VCH > 0 ? VCH : 1];
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    const int idx = threadIdx.x + NT * c;
    int row, c8;
    if constexpr (kDMA) {
      row = idx / (DK / 8);
      c8 = (idx % (DK / 8)) ^ kswz<DK>(row);   // the logical chunk stored at this position
    } else {
      row = idx / (DK / 8);
      c8 = idx % (DK / 8);
    }
    krw[c] = row;
    kgo[c] = row * kstride + c8 * 8;
    klo[c] = kchunk_off<DK>(row, c8);
  }
#pragma unroll
  for (int c = 0; c < VCH; ++c) {
    const int idx = threadIdx.x + NT * c;
    int row, c8;
    if constexpr (VL::kSwz) {
      // position idx of the V^T region: 128-byte LDS row R, chunk slot idx % 8
      constexpr int NR = VL::template rows<DV>();
      const int R = idx >> 3, cc = (idx & 7) ^ ((R >> 1) & 7);
      row = R + NR * (cc / VL::CPR);
      c8 = cc % VL::CPR;
    } else {
      row = idx / (KT / 8);
      c8 = idx % (KT / 8);
    }
    vgo[c] = row * dm.ncmp_pad + c8 * 8;
    vlo[c] = VL::template off<DV>(row, c8);
  }
  static_assert(!kDMA || VL::kSwz, "direct loads need the unpadded V^T layout");
  // the same offsets in bytes (a K tile spans KT rows of the key array, a V^T
  // tile DV rows of the padded key axis; both far below 4 GiB)
  uint32_t kgb[KCH], vgb[VCH > 0 ? VCH : 1];
#pragma unroll
  for (int c = 0; c < KCH; ++c) kgb[c] = (uint32_t)kgo[c] * (uint32_t)sizeof(T);
#pragma unroll
  for (int c = 0; c < VCH; ++c) vgb[c] = (uint32_t)vgo[c] * (uint32_t)sizeof(T);
  const int wave_pos = wave * 64;      // first position of this wave's window
  // direct-to-LDS loads of the tile at key kt into buffer buf
  // Full tiles address each chunk as the tile's (uniform) base plus the
  // thread's fixed 32-bit byte offset, the scalar-base form of the load.
  auto dma = [&](int kt, int buf) {
    T* kdst = tiles + (size_t)buf * TE;
    T* vdst = kdst + (size_t)KT * DK;
    const T* kb = kcb + (size_t)kt * kstride;
    if (kt + KT <= dm.ncmp) {
#pragma unroll
      for (int c = 0; c < KCH; ++c)
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)((const char*)kb + kgb[c]),
                                         (void __attribute__((address_space(3)))*)(kdst + (NT * c + wave_pos) * 8),
                                         16, 0, 0);
    } else {
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        // the last tile: keys past the end repeat the last key (never used)
        const int over = max(kt + krw[c] - (dm.ncmp - 1), 0);
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(kb + kgo[c] - over * kstride),
                                         (void __attribute__((address_space(3)))*)(kdst + (NT * c + wave_pos) * 8),
                                         16, 0, 0);
      }
    }
    const char* vb = (const char*)(vtb + kt);
#pragma unroll
    for (int c = 0; c < VCH; ++c)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(vb + vgb[c]),
                                       (void __attribute__((address_space(3)))*)(vdst + (NT * c + wave_pos) * 8), 16,
                                       0, 0);
  };
  auto gload = [&](int kt) {
    const T* kb = kcb + (size_t)kt * kstride;
    if (kt + KT <= dm.ncmp) {
#pragma unroll
      for (int c = 0; c < KCH; ++c) kr[c] = load_frag(kb + kgo[c]);
    } else {
      // the last tile: keys past the end repeat the last key (never used)
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int over = max(kt + krw[c] - (dm.ncmp - 1), 0);
        kr[c] = load_frag(kb + kgo[c] - over * kstride);
      }
    }
    // V^T rows are padded past the last key (zeros), so no tile needs a clamp
    const T* vb = vtb + kt;
#pragma unroll
    for (int c = 0; c < VCH; ++c) vr[c] = load_frag(vb + vgo[c]);
  };
  auto lstore = [&](int buf) {
    T* kt_ = tiles + (size_t)buf * TE;
    T* vt_ = kt_ + (size_t)KT * DK;
#pragma unroll
    for (int c = 0; c < KCH; ++c) *reinterpret_cast<Frag8<T>*>(kt_ + klo[c]) = kr[c];
#pragma unroll
    for (int c = 0; c < VCH; ++c) *reinterpret_cast<Frag8<T>*>(vt_ + vlo[c]) = vr[c];
  };

  const int krow = (c16 >> 2) * 8 + (c16 & 3);
  const int jstep = 32 * dm.d / dm.ls;
  // score-row offsets of the MFMA output rows 4*qd + r of each column tile
  // (row = position within the wave), and whether this lane writes the head
  // sum (one lane group per position once the group's heads are reduced)
  int rowoff[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) rowoff[ct][r] = ((ct * 16 + qd * 4 + r) / G) * nselp;
  const bool writer = G == 4 || (G == 8 && (qd & 1) == 0) || (G >= 16 && qd == 0);

  // scores of one 32-key half tile: S^T = K Q^T for all column tiles
  // Both MFMA blocks ask the scheduler to interleave their LDS reads with the
  // MFMAs (iglp_opt(0)); measured faster on gfx950 than its default order.
  auto scores = [&](const T* ktile, int h, f32x4 (&s)[2][NCT]) {
    __builtin_amdgcn_iglp_opt(0);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int r = h * 32 + krow + sub * 4;
      Frag8<T> kf[DK / 32];
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
        kf[ks] = *reinterpret_cast<const Frag8<T>*>(ktile + kchunk_off<DK>(r, ks * 4 + qd));
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) s[sub][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) mma(s[sub][ct], kf[ks], qf[ct][ks]);
    }
  };

  // pass A: online max / sum of exp2.  Each lane keeps its own state over the
  // keys it holds (8 of every 32) and the four lanes of a column are merged
  // once at the end, so the loop has no cross-lane traffic.  The running
  // maximum is kept raw (mr) and scaled (m, log2 units; sc2 > 0); each
  // exponent is one fma.
  auto pass_a = [&](const f32x4 (&s)[2][NCT], int kt, auto masked) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = s[e >> 2][ct][e & 3];
        if (masked) v[e] = kt + qd * 8 + e < nvis[ct] ? v[e] : kNegInf;
      }
      float mx = fmaxf(fmaxf(mr[ct], v[0]), v[1]);
      mx = fmaxf(fmaxf(mx, v[2]), v[3]);
      mx = fmaxf(fmaxf(mx, v[4]), v[5]);
      mx = fmaxf(fmaxf(mx, v[6]), v[7]);
      const float mn = mx * sc2;
      float mref = mn;
      if (masked) mref = mn == kNegInf ? 0.f : mn;   // nothing visible to this lane yet
      float acc = ls[ct] * fast_exp2(m[ct] - mref);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += fast_exp2(fmaf(v[e], sc2, -mref));
      ls[ct] = acc;
      m[ct] = mn;
      mr[ct] = mx;
    }
  };

  // pass B: exact probabilities, O += P V, remapped scores into prow
  auto pass_b = [&](const f32x4 (&s)[2][NCT], const T* vtile, int h, int kt, auto masked) {
    const int j0 = (kt / 32) * jstep;
    f32x4 cr[NCT][2];
    Frag8<T> pf[NCT], plo_all[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(fmaf(s[e >> 2][ct][e & 3], sc2, -lse2[ct]));
        if (masked) p[e] = kt + qd * 8 + e < nvis[ct] ? p[e] : 0.f;
      }
      pf[ct] = to_frag<T>(p);
      if constexpr (kSplitRemap) plo_all[ct] = lo_frag(p, pf[ct]);
      // remap onto selection blocks: P (hi + lo) times the overlap weights
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        cr[ct][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (jt < njt) {
          mma(cr[ct][jt], pf[ct], wf[jt]);
          if constexpr (kSplitRemap) mma(cr[ct][jt], plo_all[ct], wf[jt]);
        }
      }
    }
    // O^T += V^T P^T, value fragments shared by the column tiles (P as hi + lo
    // when O is kept in fp32 for the backward)
    __builtin_amdgcn_iglp_opt(0);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      const Frag8<T> vf = *reinterpret_cast<const Frag8<T>*>(vtile + VL::template off<DV>(dt * 16 + c16, h * 4 + qd));
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        mma(oacc[dt][ct], vf, pf[ct]);
        if constexpr (kPrecisePV<T, OT>) mma(oacc[dt][ct], vf, plo_all[ct]);
      }
    }
    // sum over the group's heads and accumulate the score rows in LDS
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      if (jt >= njt) break;
      const int j = j0 + jt * 16 + c16;
      if (j >= dm.nsel) continue;
      if (G >= 4) {
        float v[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) v[ct] = cr[ct][jt][0] + cr[ct][jt][1] + cr[ct][jt][2] + cr[ct][jt][3];
        if (G >= 8) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) v[ct] += xor16f(v[ct], lane);
        }
        if (G >= 16) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) v[ct] += xor32f(v[ct], lane);
        }
        if (writer) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) atomicAdd(prow + rowoff[ct][0] + j, v[ct]);
        }
      } else if (G == 2) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          prow[rowoff[ct][0] + j] += cr[ct][jt][0] + cr[ct][jt][1];
          prow[rowoff[ct][2] + j] += cr[ct][jt][2] + cr[ct][jt][3];
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) prow[rowoff[ct][r] + j] += cr[ct][jt][r];
      }
    }
  };

  const int nkt = (nmax_wg + KT - 1) / KT;
  if (nkt > 0) {
    if constexpr (kDMA) {
      dma(0, 0);
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      gload(0);
      lstore(0);
    }
  }
  __syncthreads();
  for (int it = 0; it < nkt; ++it) {
    // the next tile's loads go out first, the current tile is computed from
    // LDS, then the next tile lands in the other buffer (directly, or from
    // registers)
    const int kt0 = it * KT;
    if (it + 1 < nkt) {
      if constexpr (kDMA) dma(kt0 + KT, (it + 1) & 1);
      else gload(kt0 + KT);
    }
    const T* ktile = tiles + (size_t)(it & 1) * TE;
    const T* vtile = ktile + (size_t)KT * DK;
    // With few column tiles both halves' scores are issued before either
    // half's softmax work, so the second half's MFMAs run under the first
    // half's VALU work (four column tiles have no registers for that).
    constexpr bool kEarly = NCT <= 2 && NH == 2;
    f32x4 s[NH][2][NCT];
    if constexpr (kEarly) {
      if (kt0 < nmax) scores(ktile, 0, s[0]);
      if (kt0 + 32 < nmax) scores(ktile, 1, s[NH - 1]);
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int kt = kt0 + h * 32;
      if (kt >= nmax) break;
      if (!kEarly) scores(ktile, h, s[h]);
      const bool full = kt + 32 <= nfull;
      if constexpr (!PB) {
        if (full) pass_a(s[h], kt, std::false_type{});
        else pass_a(s[h], kt, std::true_type{});
      } else {
        if (full) pass_b(s[h], vtile, h, kt, std::false_type{});
        else pass_b(s[h], vtile, h, kt, std::true_type{});
      }
    }
    if constexpr (kDMA) {
      __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads have landed
    } else {
      if (it + 1 < nkt) lstore((it + 1) & 1);
    }
    __syncthreads();
  }
  if (!wave_live) return;
  if constexpr (!PB) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      // merge the four lane states of each column
      const float M = colmax4(m[ct], lane);
      const float part = m[ct] == kNegInf ? 0.f : ls[ct] * fast_exp2(m[ct] - M);
      const float tot = colsum4(part, lane);
      const float lse = M == kNegInf ? kNegInf : (M + __log2f(tot)) * kLn2;
      if (qd == 0 && pos[ct] < dm.T) a.lse[(size_t)(b * dm.T + pos[ct]) * dm.Hq + hq[ct]] = lse;
    }
  } else {
    // O_cmp (rows with no visible block stay 0)
    OT* o = (OT*)a.o;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (pos[ct] >= dm.T) continue;
      OT* op = o + ((size_t)(b * dm.T + pos[ct]) * dm.Hq + hq[ct]) * DV + qd * 4;
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt)
        store4(op + dt * 16, oacc[dt][ct][0], oacc[dt][ct][1], oacc[dt][ct][2], oacc[dt][ct][3]);
    }
    // top-n per position of this wave, two positions at a time
    for (int pl = 0; pl < PW; pl += 2) {
      const float* rows[2];
      int ts[2];
      int* outs[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int t = t0 + pl + r;
        const bool live = pl + r < PW && t < dm.T;
        ts[r] = live ? t : -1;
        rows[r] = prow + (pl + r) * nselp;
        const size_t rbase = (size_t)(b * dm.T + (live ? t : 0)) * dm.Hkv + g;
        outs[r] = a.idx + rbase * dm.n;
        if (live && a.p_slc) {
          float* ps = a.p_slc + rbase * dm.nsel;
          for (int j = lane; j < dm.nsel; j += 64) ps[j] = rows[r][j];
        }
      }
      if (dm.nsel <= 1024) {
        wave_topn_rows<16, 2>(rows, ts, dm.ls, dm.n, outs, lane);
      } else {
        for (int r = 0; r < 2; ++r)
          if (ts[r] >= 0) wave_topn(prow + (pl + r) * nselp, ts[r], dm.ls, dm.n, outs[r], lane);
      }
    }
  }
}

int cmp_out_nselp(const Dims& dm) { return (dm.nsel + 15) & ~15; }

template <typename T, int DK, int DV, bool PB, int KT>
static size_t cmp_lds(const Dims& dm, int nw, int nct, int nselp) {
  size_t b = 2 * cmp_tile_elems<T, DK, DV, PB, KT>() * sizeof(T);
  if (PB) b += (size_t)nw * (16 * nct / dm.G) * nselp * sizeof(float);
  return b;
}

template <typename T, int DK, int DV, int NCT, int NW, bool PB, typename OT, int KT = 64>
static hipError_t cmp_launch(const Dims& dm, const CmpArgs& a, int nselp, int njt, size_t lds, hipStream_t s) {
  // the common configuration (16 heads per group, one remap column tile) is
  // compiled with both fixed
  auto kfn = (dm.G == 16 && njt == 1 && NCT > 1) ? k_cmp<T, DK, DV, NCT, NW, PB, OT, 16, 1, KT>
                                                 : k_cmp<T, DK, DV, NCT, NW, PB, OT, 0, 0, KT>;
  if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const int PWG = NW * 16 * NCT / dm.G;
  const int ntiles = (dm.T + PWG - 1) / PWG;
  kfn<<<ntiles * dm.B * dm.Hkv, NW * 64, lds, s>>>(dm, a, nselp, njt);
  return hipGetLastError();
}

// Pass A: 4 waves x 4 column tiles, 64-key tiles.  Pass B: 4 waves x 2
// column tiles with 32-key tiles, so that two independent workgroups share a
// compute unit (two waves per SIMD that are not tied by one barrier); else 8
// waves x 2 column tiles with 64-key tiles, and with long score rows 4 waves x
// 1 column tile.
template <typename T, int DK, int DV, bool PB>
static hipError_t cmp_impl(const Dims& dm, const CmpArgs& a, hipStream_t s) {
  const int nselp = cmp_out_nselp(dm);
  const int nblk = (31 * dm.d + dm.l - 1) / dm.ls + 1;   // selection blocks one 32-key tile touches
  const int njt = (nblk + 15) / 16;
  const size_t lim = 160 * 1024;
  if constexpr (!PB) {
    const size_t lds = cmp_lds<T, DK, DV, PB, 64>(dm, 4, 4, nselp);
    return a.o_f32 ? cmp_launch<T, DK, DV, 4, 4, PB, float>(dm, a, nselp, njt, lds, s)
                   : cmp_launch<T, DK, DV, 4, 4, PB, T>(dm, a, nselp, njt, lds, s);
  } else {
  if (2 * cmp_lds<T, DK, DV, PB, 32>(dm, 4, 2, nselp) <= lim) {
    const size_t lds = cmp_lds<T, DK, DV, PB, 32>(dm, 4, 2, nselp);
    return a.o_f32 ? cmp_launch<T, DK, DV, 2, 4, PB, float, 32>(dm, a, nselp, njt, lds, s)
                   : cmp_launch<T, DK, DV, 2, 4, PB, T, 32>(dm, a, nselp, njt, lds, s);
  }
  if (cmp_lds<T, DK, DV, PB, 64>(dm, 8, 2, nselp) <= lim) {
    const size_t lds = cmp_lds<T, DK, DV, PB, 64>(dm, 8, 2, nselp);
    return a.o_f32 ? cmp_launch<T, DK, DV, 2, 8, PB, float>(dm, a, nselp, njt, lds, s)
                   : cmp_launch<T, DK, DV, 2, 8, PB, T>(dm, a, nselp, njt, lds, s);
  }
  const size_t lds = cmp_lds<T, DK, DV, PB, 64>(dm, 4, 1, nselp);
  if (lds > lim) return hipErrorInvalidValue;
  return a.o_f32 ? cmp_launch<T, DK, DV, 1, 4, PB, float>(dm, a, nselp, njt, lds, s)
                 : cmp_launch<T, DK, DV, 1, 4, PB, T>(dm, a, nselp, njt, lds, s);
  }
}

template <bool PB>
static hipError_t cmp_dispatch(const Dims& dm, const CmpArgs& a, hipStream_t s) {
  const bool bf = dm.io == IO_BF16;
  if (dm.dk == 64 && dm.dv == 64) return bf ? cmp_impl<bf16, 64, 64, PB>(dm, a, s) : cmp_impl<float, 64, 64, PB>(dm, a, s);
  if (dm.dk == 128 && dm.dv == 128) return bf ? cmp_impl<bf16, 128, 128, PB>(dm, a, s) : cmp_impl<float, 128, 128, PB>(dm, a, s);
  if (dm.dk == 192 && dm.dv == 128) return bf ? cmp_impl<bf16, 192, 128, PB>(dm, a, s) : cmp_impl<float, 192, 128, PB>(dm, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_cmp_lse(const Dims& dm, const CmpArgs& a, hipStream_t s) { return cmp_dispatch<false>(dm, a, s); }
hipError_t launch_cmp_out_topn(const Dims& dm, const CmpArgs& a, hipStream_t s) { return cmp_dispatch<true>(dm, a, s); }

bool cmp_out_fits(const Dims& dm) {
  // pass B with one column tile per wave: tiles (largest case: fp32, 192/128) + score rows
  const size_t tiles = 2 * ((size_t)64 * dm.dk + (size_t)dm.dv * cmp_vs<64>()) * (dm.io == IO_BF16 ? 2 : 4);  // an upper bound
  return tiles + (size_t)4 * (16 / dm.G) * cmp_out_nselp(dm) * sizeof(float) <= 160 * 1024;
}

}  // namespace nsa
