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
// matrix, with P split into bf16 hi + lo parts so the scores keep ~16
// significant bits), sums over heads with cross-lane adds, keeps each
// position's score row in LDS and runs the top-n selection there.
//
// Layout of the work: a wave owns 16*NCT query columns = (positions x G heads
// of one KV group); MFMA tiles compute S^T = K Q^T (16 keys x 16 columns) so
// that every lane holds one column's scores for 8 keys, which is directly the
// B operand of O^T = V^T P^T.  Keys inside a 32-key tile are permuted so that
// lane group qd (= lane/16) ends up holding keys 8*qd .. 8*qd+7.
#include "nsa_common.hpp"
#include "nsa_kernels.hpp"

namespace nsa {

template <typename T, int DK, int NCT>
__global__ __launch_bounds__(256) void k_cmp_lse(Dims dm, CmpArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  const int G = dm.G, PW = 16 * NCT / G, PWG = 4 * PW;
  const int ntiles = (dm.T + PWG - 1) / PWG;
  int unit, tile;
  xcd_map(blockIdx.x, dm.B * dm.Hkv, ntiles, unit, tile);
  const int b = unit / dm.Hkv, g = unit % dm.Hkv;
  const int t0 = tile * PWG + wave * PW;
  if (t0 >= dm.T) return;
  const int tl = min(dm.T - 1, t0 + PW - 1);
  const int nmax = ncmp_visible(tl, dm.l, dm.d);
  const T* q = (const T*)a.q;
  Frag8<T> qf[NCT][DK / 32];
  int pos[NCT], hq[NCT], nvis[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = ct * 16 + c16;
    pos[ct] = t0 + col / G;
    hq[ct] = g * G + col % G;
    const bool v = pos[ct] < dm.T;
    nvis[ct] = v ? ncmp_visible(pos[ct], dm.l, dm.d) : 0;
    const T* qp = q + ((size_t)(b * dm.T + min(pos[ct], dm.T - 1)) * dm.Hq + hq[ct]) * DK + qd * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qf[ct][ks] = v ? load_frag(qp + ks * 32) : zero_frag<T>();
  }
  const float sc2 = dm.scale * kLog2e;
  float m[NCT], ls[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) { m[ct] = kNegInf; ls[ct] = 0.f; }
  const size_t kstride = (size_t)dm.Hkv * DK;
  const T* kbase = (const T*)a.kc + ((size_t)b * dm.ncmp * dm.Hkv + g) * DK + qd * 8;
  const int krow = (c16 >> 2) * 8 + (c16 & 3);
  for (int kt = 0; kt < nmax; kt += 32) {
    f32x4 s[2][NCT];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) s[sub][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = min(kt + krow + sub * 4, dm.ncmp - 1);
      const T* kp = kbase + (size_t)key * kstride;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        Frag8<T> kf = load_frag(kp + ks * 32);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) mma(s[sub][ct], kf, qf[ct][ks]);
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float v[8], mx = kNegInf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kt + qd * 8 + e;
        v[e] = key < nvis[ct] ? s[e >> 2][ct][e & 3] * sc2 : kNegInf;
        mx = fmaxf(mx, v[e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m[ct], mx);
      const float mref = mn == kNegInf ? 0.f : mn;
      float acc = ls[ct] * fast_exp2(m[ct] - mref);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += fast_exp2(v[e] - mref);
      ls[ct] = acc;
      m[ct] = mn;
    }
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    float tot = ls[ct] + __shfl_xor(ls[ct], 16);
    tot += __shfl_xor(tot, 32);
    const float lse = m[ct] == kNegInf ? kNegInf : (m[ct] + __log2f(tot)) * kLn2;
    if (qd == 0 && pos[ct] < dm.T) a.lse[(size_t)(b * dm.T + pos[ct]) * dm.Hq + hq[ct]] = lse;
  }
}

template <typename T, int DK, int DV, int NCT, typename OT>
__global__ __launch_bounds__(256) void k_cmp_out(Dims dm, CmpArgs a, int nselp, int njt) {
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  const int G = dm.G, PW = 16 * NCT / G, PWG = 4 * PW;
  const int ntiles = (dm.T + PWG - 1) / PWG;
  int unit, tile;
  xcd_map(blockIdx.x, dm.B * dm.Hkv, ntiles, unit, tile);
  const int b = unit / dm.Hkv, g = unit % dm.Hkv;
  const int t0 = tile * PWG + wave * PW;
  if (t0 >= dm.T) return;
  float* prow = smem + (size_t)wave * PW * nselp;
  for (int i = lane; i < PW * nselp; i += 64) prow[i] = 0.f;

  const int tl = min(dm.T - 1, t0 + PW - 1);
  const int nmax = ncmp_visible(tl, dm.l, dm.d);
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
    lse2[ct] = (v && nvis[ct] > 0) ? a.lse[row] * kLog2e : 0.f;
    const T* qp = q + row * DK + qd * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qf[ct][ks] = v ? load_frag(qp + ks * 32) : zero_frag<T>();
  }
  // remap matrix fragments (constant over tiles since l' divides 32*d)
  Frag8<T> wf[2];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = jt < njt ? remap_weight(qd * 8 + e, jt * 16 + c16, dm.l, dm.d, dm.ls) : 0.f;
    wf[jt] = to_frag<T>(w);
  }
  const float sc2 = dm.scale * kLog2e;
  f32x4 oacc[DV / 16][NCT];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) oacc[dt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  const size_t kstride = (size_t)dm.Hkv * DK;
  const T* kbase = (const T*)a.kc + ((size_t)b * dm.ncmp * dm.Hkv + g) * DK + qd * 8;
  const T* vtb = (const T*)a.vct + (size_t)(b * dm.Hkv + g) * DV * dm.ncmp_pad + qd * 8;
  const int krow = (c16 >> 2) * 8 + (c16 & 3);
  const int jstep = 32 * dm.d / dm.ls;
  for (int kt = 0; kt < nmax; kt += 32) {
    f32x4 s[2][NCT];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) s[sub][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = min(kt + krow + sub * 4, dm.ncmp - 1);
      const T* kp = kbase + (size_t)key * kstride;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        Frag8<T> kf = load_frag(kp + ks * 32);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) mma(s[sub][ct], kf, qf[ct][ks]);
      }
    }
    Frag8<T> vf[DV / 16];
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) vf[dt] = load_frag(vtb + (size_t)(dt * 16 + c16) * dm.ncmp_pad + kt);
    const int j0 = (kt / 32) * jstep;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kt + qd * 8 + e;
        p[e] = key < nvis[ct] ? fast_exp2(s[e >> 2][ct][e & 3] * sc2 - lse2[ct]) : 0.f;
      }
      Frag8<T> pf = to_frag<T>(p);
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) mma(oacc[dt][ct], vf[dt], pf);
      // remap onto selection blocks and sum over the group's heads
      Frag8<T> phi = pf, plo;
      if constexpr (sizeof(T) == 2) split_bf16(p, phi, plo);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        if (jt >= njt) break;
        f32x4 cr = f32x4{0.f, 0.f, 0.f, 0.f};
        mma(cr, phi, wf[jt]);
        if constexpr (sizeof(T) == 2) mma(cr, plo, wf[jt]);
        const int j = j0 + jt * 16 + c16;
        const int col = ct * 16 + qd * 4;
        if (G >= 4) {
          float v = cr[0] + cr[1] + cr[2] + cr[3];
          if (G >= 8) v += __shfl_xor(v, 16);
          if (G >= 16) v += __shfl_xor(v, 32);
          const bool writer = G == 4 || (G == 8 && (qd & 1) == 0) || (G >= 16 && qd == 0);
          if (writer && j < dm.nsel) prow[(col / G) * nselp + j] += v;
        } else if (G == 2) {
          if (j < dm.nsel) {
            prow[(col / 2) * nselp + j] += cr[0] + cr[1];
            prow[(col / 2 + 1) * nselp + j] += cr[2] + cr[3];
          }
        } else {
          if (j < dm.nsel)
#pragma unroll
            for (int r = 0; r < 4; ++r) prow[(col + r) * nselp + j] += cr[r];
        }
      }
    }
  }
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
  // top-n per position of this wave
  const int n = dm.n;
  for (int pl = 0; pl < PW; ++pl) {
    const int t = t0 + pl;
    if (t >= dm.T) break;
    float* row = prow + pl * nselp;
    const size_t rbase = (size_t)(b * dm.T + t) * dm.Hkv + g;
    if (a.p_slc) {
      float* ps = a.p_slc + rbase * dm.nsel;
      for (int j = lane; j < dm.nsel; j += 64) ps[j] = row[j];
    }
    wave_topn(row, t, dm.ls, n, a.idx + rbase * n, lane);
  }
}

template <typename T, int DK>
static hipError_t cmp_lse_impl(const Dims& dm, const CmpArgs& a, hipStream_t s) {
  constexpr int NCT = 4;
  const int PWG = 4 * 16 * NCT / dm.G;
  const int ntiles = (dm.T + PWG - 1) / PWG;
  k_cmp_lse<T, DK, NCT><<<ntiles * dm.B * dm.Hkv, 256, 0, s>>>(dm, a);
  return hipGetLastError();
}

hipError_t launch_cmp_lse(const Dims& dm, const CmpArgs& a, hipStream_t s) {
  const bool bf = dm.io == IO_BF16;
  switch (dm.dk) {
    case 64: return bf ? cmp_lse_impl<bf16, 64>(dm, a, s) : cmp_lse_impl<float, 64>(dm, a, s);
    case 128: return bf ? cmp_lse_impl<bf16, 128>(dm, a, s) : cmp_lse_impl<float, 128>(dm, a, s);
    case 192: return bf ? cmp_lse_impl<bf16, 192>(dm, a, s) : cmp_lse_impl<float, 192>(dm, a, s);
  }
  return hipErrorInvalidValue;
}

// LDS bytes pass B needs with NCT column tiles per wave.
static size_t cmp_out_lds(const Dims& dm, int nct, int nselp) {
  return (size_t)4 * (16 * nct / dm.G) * nselp * sizeof(float);
}

int cmp_out_nselp(const Dims& dm) { return (dm.nsel + 15) & ~15; }

template <typename T, int DK, int DV>
static hipError_t cmp_out_impl(const Dims& dm, const CmpArgs& a, hipStream_t s) {
  const int nselp = cmp_out_nselp(dm);
  const int nblk = (31 * dm.d + dm.l - 1) / dm.ls + 1;   // selection blocks one key tile touches
  const int njt = (nblk + 15) / 16;
  const size_t lim = 160 * 1024;
  int nct = cmp_out_lds(dm, 4, nselp) <= lim ? 4 : 1;
  const size_t lds = cmp_out_lds(dm, nct, nselp);
  if (lds > lim) return hipErrorInvalidValue;
  const int PWG = 4 * 16 * nct / dm.G;
  const int ntiles = (dm.T + PWG - 1) / PWG;
  if (nct == 4) {
    auto kfn = a.o_f32 ? k_cmp_out<T, DK, DV, 4, float> : k_cmp_out<T, DK, DV, 4, T>;
    if (lds > 64 * 1024) hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    kfn<<<ntiles * dm.B * dm.Hkv, 256, lds, s>>>(dm, a, nselp, njt);
  } else {
    auto kfn = a.o_f32 ? k_cmp_out<T, DK, DV, 1, float> : k_cmp_out<T, DK, DV, 1, T>;
    if (lds > 64 * 1024) hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    kfn<<<ntiles * dm.B * dm.Hkv, 256, lds, s>>>(dm, a, nselp, njt);
  }
  return hipGetLastError();
}

hipError_t launch_cmp_out_topn(const Dims& dm, const CmpArgs& a, hipStream_t s) {
  const bool bf = dm.io == IO_BF16;
  if (dm.dk == 64 && dm.dv == 64) return bf ? cmp_out_impl<bf16, 64, 64>(dm, a, s) : cmp_out_impl<float, 64, 64>(dm, a, s);
  if (dm.dk == 128 && dm.dv == 128) return bf ? cmp_out_impl<bf16, 128, 128>(dm, a, s) : cmp_out_impl<float, 128, 128>(dm, a, s);
  if (dm.dk == 192 && dm.dv == 128) return bf ? cmp_out_impl<bf16, 192, 128>(dm, a, s) : cmp_out_impl<float, 192, 128>(dm, a, s);
  return hipErrorInvalidValue;
}

bool cmp_out_fits(const Dims& dm) {
  return cmp_out_lds(dm, 1, cmp_out_nselp(dm)) <= 160 * 1024;
}

}  // namespace nsa
