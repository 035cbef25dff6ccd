// Gate projection, layout transposes and token compression phi (mean-pool or
// MLP with intra-block position embedding) for gfx950.
//
// Compression (youleyou NSA page, 令牌压缩): block i covers tokens
// [i*d, i*d+l); phi maps the block to one key (value).  The MLP variant is
//     phi(block i) = gelu(u_i w1 + b1) w2 + b2,  u_i = concat_j (x[i*d+j] + pe[j]).
// Because the stride d divides l, u_i is the concatenation of l/d stride-sized
// sub-blocks s_{i}, s_{i+1}, ..., so
//     u_i w1 = sum_r s_{i+r} w1_r + sum_r pe_r w1_r,
// where w1_r are the l/d row chunks of w1.  The first GEMM therefore multiplies
// every sub-block once by every chunk (instead of materialising the
// overlapping blocks), and the constant pe term comes out of the same GEMM as
// l/d extra rows.
#include "nsa_common.hpp"
#include "nsa_kernels.hpp"

namespace nsa {

// ---------------------------------------------------------------------------
// Gate layers, fp32 math: out[tok, o] = act(sum_i x[tok,i] w[i, o] + bias[o]),
// act = identity (0), exact GELU (1) or sigmoid (2); `pre` (optional) receives
// the value before the activation.  One linear layer with a sigmoid gives the
// gates g = sigmoid(x W_g); the gate MLP is a GELU layer followed by it.
// ---------------------------------------------------------------------------
template <typename TX, typename TW, int ACT>
__global__ __launch_bounds__(256) void k_gate(int ntok, int C, int HO, const TX* __restrict__ x,
                                              const TW* __restrict__ w, const TW* __restrict__ bias,
                                              float* __restrict__ out, float* __restrict__ pre) {
  constexpr int TOK = 16;
  extern __shared__ float xs[];
  const int tok0 = blockIdx.x * TOK;
  for (int i = threadIdx.x; i < TOK * C; i += blockDim.x) {
    int tk = i / C, c = i % C;
    xs[i] = (tok0 + tk < ntok) ? to_f32(x[(size_t)(tok0 + tk) * C + c]) : 0.f;
  }
  __syncthreads();
  for (int oc = threadIdx.x; oc < HO; oc += blockDim.x) {
    const float b0 = bias ? to_f32(bias[oc]) : 0.f;
    float acc[TOK];
#pragma unroll
    for (int tk = 0; tk < TOK; ++tk) acc[tk] = b0;
    for (int i = 0; i < C; ++i) {
      float wv = to_f32(w[(size_t)i * HO + oc]);
#pragma unroll
      for (int tk = 0; tk < TOK; ++tk) acc[tk] = fmaf(xs[tk * C + i], wv, acc[tk]);
    }
#pragma unroll
    for (int tk = 0; tk < TOK; ++tk) {
      if (tok0 + tk >= ntok) continue;
      const size_t o = (size_t)(tok0 + tk) * HO + oc;
      const float a = acc[tk];
      if (pre) pre[o] = a;
      out[o] = ACT == 2 ? 1.f / (1.f + expf(-a)) : (ACT == 1 ? 0.5f * a * (1.f + erff(a * 0.70710678118654752f)) : a);
    }
  }
}

template <typename TX, typename TW, int ACT>
static hipError_t gate_layer(int ntok, int C, int HO, const void* x, const void* w, const void* bias, float* out,
                             float* pre, hipStream_t s) {
  dim3 grid((ntok + 15) / 16);
  k_gate<TX, TW, ACT><<<grid, 256, 16 * C * sizeof(float), s>>>(ntok, C, HO, (const TX*)x, (const TW*)w,
                                                                 (const TW*)bias, out, pre);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_sigmoid(size_t n, float* __restrict__ g) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) g[i] = 1.f / (1.f + expf(-g[i]));
}

// The linear gate: with bf16 I/O a bf16 MFMA GEMM (fp32 accumulation and
// output), then the sigmoid in place; fp32 I/O, or a gate width the GEMM's
// 16-byte loads cannot take, runs the fp32 gate layer.
hipError_t launch_gate(const Dims& dm, int ntok, const void* x, const void* w, float* gates,
                       hipStream_t s) {
  const int HO = dm.Hq * 3;
  if (ntok == 0) return hipSuccess;
  if (dm.io == IO_BF16) {
    const MmArgs g{ntok, HO, dm.C, x, dm.C, 1, w, HO, 1, gates, HO, 0, 0};
    if (mm_supported(g, false, false)) {
      hipError_t e = mm(g, false, false, 1, nullptr, s);
      if (e != hipSuccess) return e;
      const size_t n = (size_t)ntok * HO;
      k_sigmoid<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(n, gates);
      return hipGetLastError();
    }
    return gate_layer<bf16, bf16, 2>(ntok, dm.C, HO, x, w, nullptr, gates, nullptr, s);
  }
  return gate_layer<float, float, 2>(ntok, dm.C, HO, x, w, nullptr, gates, nullptr, s);
}

hipError_t launch_gate_mlp(const Dims& dm, int ntok, const void* x, const void* w_gate, const GateMlp& g,
                           float* hid, float* pre, float* gates, hipStream_t s) {
  if (dm.Cg == 0) return launch_gate(dm, ntok, x, w_gate, gates, s);
  const int HO = dm.Hq * 3;
  hipError_t e;
  if (dm.io == IO_BF16) {
    if ((e = gate_layer<bf16, bf16, 1>(ntok, dm.C, dm.Cg, x, g.w1, g.b1, hid, pre, s)) != hipSuccess) return e;
    return gate_layer<float, bf16, 2>(ntok, dm.Cg, HO, hid, w_gate, g.b2, gates, nullptr, s);
  }
  if ((e = gate_layer<float, float, 1>(ntok, dm.C, dm.Cg, x, g.w1, g.b1, hid, pre, s)) != hipSuccess) return e;
  return gate_layer<float, float, 2>(ntok, dm.Cg, HO, hid, w_gate, g.b2, gates, nullptr, s);
}

__global__ __launch_bounds__(256) void k_to_f32(size_t n, const bf16* __restrict__ src, float* __restrict__ dst) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i + 8 <= n) {
    const Frag8<bf16> f = load_frag(src + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[i + e] = to_f32(frag_at(f, e));
  } else {
    for (size_t j = i; j < n; ++j) dst[j] = to_f32(src[j]);
  }
}

hipError_t launch_to_f32(const void* src, size_t n, float* dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  k_to_f32<<<(unsigned)((n + 2047) / 2048), 256, 0, s>>>(n, (const bf16*)src, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Transposes.
// ---------------------------------------------------------------------------
// src [B, n, H, D] -> dst [B, H, D, ldd]; zeros in columns n .. ldd-1.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose_seq(int n, int H, int D, int ldd,
                                                       const T* __restrict__ src, T* __restrict__ dst) {
  __shared__ float tile[64][65];
  const int bh = blockIdx.z, b = bh / H, h = bh % H;
  const int t0 = blockIdx.x * 64, f0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    int tt = i >> 6, ff = i & 63, t = t0 + tt, f = f0 + ff;
    tile[tt][ff] = (t < n && f < D) ? to_f32(src[((size_t)(b * n + t) * H + h) * D + f]) : 0.f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    int ff = i >> 6, tt = i & 63, t = t0 + tt, f = f0 + ff;
    if (f < D && t < ldd) dst[((size_t)(b * H + h) * D + f) * ldd + t] = from_f32<T>(tile[tt][ff]);
  }
}

hipError_t launch_transpose_seq(const Dims& dm, int B, int n, int H, int D, int ldd,
                                const void* src, void* dst, hipStream_t s) {
  dim3 grid((ldd + 63) / 64, (D + 63) / 64, B * H);
  if (dm.io == IO_BF16)
    k_transpose_seq<bf16><<<grid, 256, 0, s>>>(n, H, D, ldd, (const bf16*)src, (bf16*)dst);
  else
    k_transpose_seq<float><<<grid, 256, 0, s>>>(n, H, D, ldd, (const float*)src, (float*)dst);
  return hipGetLastError();
}

// src [R, Cc] -> dst [Cc, R]
template <typename T>
__global__ __launch_bounds__(256) void k_transpose_2d(int R, int Cc, const T* __restrict__ src,
                                                      T* __restrict__ dst) {
  __shared__ float tile[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    int rr = i >> 6, cc = i & 63, r = r0 + rr, c = c0 + cc;
    tile[rr][cc] = (r < R && c < Cc) ? to_f32(src[(size_t)r * Cc + c]) : 0.f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    int cc = i >> 6, rr = i & 63, r = r0 + rr, c = c0 + cc;
    if (r < R && c < Cc) dst[(size_t)c * R + r] = from_f32<T>(tile[rr][cc]);
  }
}

hipError_t launch_transpose_2d(const Dims& dm, int R, int Cc, const void* src, void* dst,
                               hipStream_t s) {
  dim3 grid((R + 63) / 64, (Cc + 63) / 64);
  if (dm.io == IO_BF16)
    k_transpose_2d<bf16><<<grid, 256, 0, s>>>(R, Cc, (const bf16*)src, (bf16*)dst);
  else
    k_transpose_2d<float><<<grid, 256, 0, s>>>(R, Cc, (const float*)src, (float*)dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Mean-pool compression: out[b,i,g,:] = (1/l) sum_{j<l} x[b, i*d+j, g, :].
// One thread per (b, i, g, 8-feature chunk); i runs to ncmp_pad so that the
// transposed copy's padding columns are written as zeros.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_meanpool(Dims dm, int D, const T* __restrict__ x,
                                                  T* __restrict__ out, T* __restrict__ outT) {
  const int chunks = D / 8;
  const size_t total = (size_t)dm.B * dm.ncmp_pad * dm.Hkv * chunks;
  size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= total) return;
  int c = id % chunks;
  size_t r = id / chunks;
  int g = r % dm.Hkv;
  r /= dm.Hkv;
  int i = r % dm.ncmp_pad;
  int b = r / dm.ncmp_pad;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (i < dm.ncmp) {
    const T* p = x + ((size_t)(b * dm.T + i * dm.d) * dm.Hkv + g) * D + c * 8;
    for (int j = 0; j < dm.l; ++j) {
      Frag8<T> f = load_frag(p + (size_t)j * dm.Hkv * D);
      float v[8];
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)f.v[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = f.lo[e]; v[4 + e] = f.hi[e]; }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] / (float)dm.l;
    T* o = out + ((size_t)(b * dm.ncmp + i) * dm.Hkv + g) * D + c * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(acc[e]);
  }
  if (outT) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      outT[((size_t)(b * dm.Hkv + g) * D + c * 8 + e) * dm.ncmp_pad + i] = from_f32<T>(acc[e]);
  }
}

hipError_t launch_meanpool(const Dims& dm, int D, const void* x, void* out, void* outT,
                           hipStream_t s) {
  size_t total = (size_t)dm.B * dm.ncmp_pad * dm.Hkv * (D / 8);
  dim3 grid((unsigned)((total + 255) / 256));
  if (total == 0) return hipSuccess;
  if (dm.io == IO_BF16)
    k_meanpool<bf16><<<grid, 256, 0, s>>>(dm, D, (const bf16*)x, (bf16*)out, (bf16*)outT);
  else
    k_meanpool<float><<<grid, 256, 0, s>>>(dm, D, (const float*)x, (float*)out, (float*)outT);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MLP compression.
//   GEMM1: y[m, r*H + o] = sum_x A[m, x] * w1[r*d*D + x, o]   (x < d*D)
//          rows m < Mmain: stride sub-block s of (b, g): A[m, j*D + e] = x[b, s*d + j, g, e]
//          rows Mmain + r: A = pe rows r*d .. r*d+d-1 (flattened)
//   hidden: a = b1 + sum_r y[Mmain + r, r*H + o] + sum_r y[(bg, i + r), r*H + o]; h = gelu(a)
//   GEMM2: out[b, i, g, :] = h w2 + b2, rounded to the I/O type.
// GEMM1 is a plain dense GEMM once the rows of A are laid out contiguously
// (k_phi_arows): one bf16 MFMA GEMM per W1 chunk r (nsa_gemm.hip), fp32
// accumulation and output.  GEMM2 (small) is k_phi_gemm2: each wave owns a
// 32x32 output tile (2x2 MFMA 16x16 tiles), a workgroup of four waves 64x64.
// ---------------------------------------------------------------------------
// A rows: sub-block s of (b, g) as d*D contiguous elements, then the R
// position-embedding rows (pe rows r*d .. r*d+d-1).  8 elements per thread.
template <typename T>
__global__ __launch_bounds__(256) void k_phi_arows(Dims dm, int D, int nsub, const T* __restrict__ x,
                                                   const T* __restrict__ pe, T* __restrict__ arows) {
  const int KK = dm.d * D, R = dm.l / dm.d;
  const size_t Mmain = (size_t)dm.B * dm.Hkv * nsub;
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (Mmain + R) * (KK / 8)) return;
  const size_t m = id / (KK / 8);
  const int k = (int)(id % (KK / 8)) * 8;
  const T* src;
  if (m < Mmain) {
    const int bg = (int)(m / nsub), sidx = (int)(m % nsub), b = bg / dm.Hkv, g = bg % dm.Hkv;
    const int j = k / D, e = k % D;
    src = x + ((size_t)(b * dm.T + sidx * dm.d + j) * dm.Hkv + g) * D + e;
  } else {
    src = pe + (size_t)(m - Mmain) * KK + k;
  }
  *reinterpret_cast<Frag8<T>*>(arows + m * KK + k) = load_frag(src);
}


// The position-embedding rows of y: y[Mmain + r, r*H + o] = pe_r . W1_r[:, o]
// (pe_r: the d rows of pe that chunk r covers, KK = d*D values), the same
// for every block.  Stage 1: workgroup (o chunk of 64, r, slice z) sums the
// kPeSlices-th part z of the KK products, four waves a quarter of it each;
// stage 2 adds the slices in order (deterministic, no atomics).
constexpr int kPeSlices = 16;

size_t phi_pe_part_floats(const Dims& dm) { return (size_t)kPeSlices * (dm.l / dm.d) * dm.hidden; }

template <typename T>
__global__ __launch_bounds__(256) void k_phi_pe_part(Dims dm, int D, const T* __restrict__ pe,
                                                     const T* __restrict__ w1, float* __restrict__ part) {
  __shared__ float red[4][64];
  const int H = dm.hidden, KK = dm.d * D;
  const int r = blockIdx.y, z = blockIdx.z, o = blockIdx.x * 64 + (threadIdx.x & 63), q = threadIdx.x >> 6;
  const int len = (KK + kPeSlices * 4 - 1) / (kPeSlices * 4);
  const int k0 = (z * 4 + q) * len, k1 = min(KK, k0 + len);
  float s = 0.f;
  if (o < H) {
#pragma unroll 8
    for (int k = k0; k < k1; ++k)
      s = fmaf(to_f32(pe[(size_t)r * KK + k]), to_f32(w1[((size_t)r * KK + k) * H + o]), s);
  }
  red[q][threadIdx.x & 63] = s;
  __syncthreads();
  if (q == 0 && o < H) {
    const int t = threadIdx.x;
    part[((size_t)r * kPeSlices + z) * H + o] = red[0][t] + red[1][t] + red[2][t] + red[3][t];
  }
}

__global__ __launch_bounds__(256) void k_phi_pe_fin(Dims dm, size_t Mmain, const float* __restrict__ part,
                                                    float* __restrict__ y) {
  const int H = dm.hidden, R = dm.l / dm.d;
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id >= R * H) return;
  const int r = id / H, o = id % H;
  float s = 0.f;
  for (int z = 0; z < kPeSlices; ++z) s += part[((size_t)r * kPeSlices + z) * H + o];
  y[(Mmain + r) * (size_t)(R * H) + (size_t)r * H + o] = s;
}

// h rows: (b*Hkv + g)*ncmp + i.  bf16 I/O: h holds hi rows then lo rows (bf16);
// fp32 I/O: h is fp32.
template <typename T>
__global__ __launch_bounds__(256) void k_phi_hidden(Dims dm, int nsub, const float* __restrict__ y,
                                                    const T* __restrict__ b1, void* __restrict__ h) {
  const int H = dm.hidden, R = dm.l / dm.d, N = R * H;
  const size_t rows = (size_t)dm.B * dm.Hkv * dm.ncmp;
  size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * H) return;
  int o = id % H;
  size_t row = id / H;
  int i = row % dm.ncmp;
  size_t bg = row / dm.ncmp;
  const size_t Mmain = (size_t)dm.B * dm.Hkv * nsub;
  float a = to_f32(b1[o]);
  for (int r = 0; r < R; ++r) a += y[(Mmain + r) * N + (size_t)r * H + o];
  for (int r = 0; r < R; ++r) a += y[(bg * nsub + i + r) * N + (size_t)r * H + o];
  float gl = 0.5f * a * (1.f + erff(a * 0.70710678118654752f));
  if constexpr (sizeof(T) == 2) {
    bf16 hi = (bf16)gl;
    bf16 lo = (bf16)(gl - (float)hi);
    ((bf16*)h)[row * H + o] = hi;
    ((bf16*)h)[(rows + row) * H + o] = lo;
  } else {
    ((float*)h)[row * H + o] = gl;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_phi_gemm2(Dims dm, const void* __restrict__ h,
                                                   const T* __restrict__ w2t, const T* __restrict__ b2,
                                                   T* __restrict__ out, T* __restrict__ outT) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  const int H = dm.hidden;
  const int M = dm.B * dm.Hkv * dm.ncmp;
  const int mbase = blockIdx.y * 64 + (wave >> 1) * 32;
  const int nbase = blockIdx.x * 64 + (wave & 1) * 32;
  f32x4 acc[2][2];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int mrow[2];
  for (int i = 0; i < 2; ++i) mrow[i] = min(mbase + i * 16 + c16, M - 1);
  int ncol[2];
  for (int j = 0; j < 2; ++j) ncol[j] = min(nbase + j * 16 + c16, D - 1);
  for (int kk = 0; kk < H; kk += 32) {
    const int xx = kk + qd * 8;
    Frag8<T> bfr[2];
    for (int j = 0; j < 2; ++j) bfr[j] = load_frag(w2t + (size_t)ncol[j] * H + xx);
    if constexpr (sizeof(T) == 2) {
      const bf16* hh = (const bf16*)h;
      for (int i = 0; i < 2; ++i) {
        Frag8<bf16> ahi = load_frag(hh + (size_t)mrow[i] * H + xx);
        Frag8<bf16> alo = load_frag(hh + ((size_t)M + mrow[i]) * H + xx);
        for (int j = 0; j < 2; ++j) {
          mma(acc[i][j], ahi, bfr[j]);
          mma(acc[i][j], alo, bfr[j]);
        }
      }
    } else {
      const float* hh = (const float*)h;
      for (int i = 0; i < 2; ++i) {
        Frag8<float> a = load_frag(hh + (size_t)mrow[i] * H + xx);
        for (int j = 0; j < 2; ++j) mma(acc[i][j], a, bfr[j]);
      }
    }
  }
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) {
      int n = nbase + j * 16 + c16;
      if (n >= D) continue;
      float bias = to_f32(b2[n]);
      for (int r = 0; r < 4; ++r) {
        int m = mbase + i * 16 + qd * 4 + r;
        if (m >= M) continue;
        int ii = m % dm.ncmp, bg = m / dm.ncmp, g = bg % dm.Hkv, b = bg / dm.Hkv;
        T v = from_f32<T>(acc[i][j][r] + bias);
        out[((size_t)(b * dm.ncmp + ii) * dm.Hkv + g) * D + n] = v;
        if (outT) outT[((size_t)(b * dm.Hkv + g) * D + n) * dm.ncmp_pad + ii] = v;
      }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_zero_tail(Dims dm, int D, T* __restrict__ outT) {
  // zero columns ncmp .. ncmp_pad-1 of outT [B*Hkv*D, ncmp_pad]
  const int padw = dm.ncmp_pad - dm.ncmp;
  size_t total = (size_t)dm.B * dm.Hkv * D * padw;
  size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= total) return;
  size_t row = id / padw;
  int c = dm.ncmp + id % padw;
  outT[row * dm.ncmp_pad + c] = from_f32<T>(0.f);
}

size_t phi_mlp_ws_bytes(const Dims& dm, int D) {
  const int R = dm.l / dm.d;
  const size_t es = dm.io == IO_BF16 ? 2 : 4;
  const int nsub = dm.ncmp > 0 ? dm.ncmp + R - 1 : 0;
  size_t b = 0;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  b += al(((size_t)dm.B * dm.Hkv * nsub + R) * dm.d * D * es);      // arows
  b += al((size_t)D * dm.hidden * es);                              // w2t
  b += al(phi_pe_part_floats(dm) * 4);                              // pe-row partial sums
  b += al(((size_t)dm.B * dm.Hkv * nsub + R) * R * dm.hidden * 4);  // y
  b += al((size_t)dm.B * dm.Hkv * dm.ncmp * dm.hidden * (dm.io == IO_BF16 ? 4 : 4));  // h
  return b;
}

template <typename T, int D>
static hipError_t phi_mlp_impl(const Dims& dm, const PhiMlpArgs& a, hipStream_t s) {
  const int R = dm.l / dm.d;
  const int nsub = dm.ncmp + R - 1;
  hipError_t e;
  if ((e = launch_transpose_2d(dm, dm.hidden, D, a.w2, a.w2t, s)) != hipSuccess) return e;
  if ((e = launch_phi_gemm1(dm, D, nsub, a.x, a.pe, a.w1, a.arows, a.y, a.pe_part, s)) != hipSuccess) return e;
  {
    size_t total = (size_t)dm.B * dm.Hkv * dm.ncmp * dm.hidden;
    k_phi_hidden<T><<<(unsigned)((total + 255) / 256), 256, 0, s>>>(dm, nsub, a.y, (const T*)a.b1, a.h);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    const int M = dm.B * dm.Hkv * dm.ncmp;
    dim3 grid((D + 63) / 64, (M + 63) / 64);
    k_phi_gemm2<T, D><<<grid, 256, 0, s>>>(dm, a.h, (const T*)a.w2t, (const T*)a.b2, (T*)a.out, (T*)a.outT);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.outT) {
    size_t total = (size_t)dm.B * dm.Hkv * D * (dm.ncmp_pad - dm.ncmp);
    k_zero_tail<T><<<(unsigned)((total + 255) / 256), 256, 0, s>>>(dm, D, (T*)a.outT);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_phi_gemm1(const Dims& dm, int D, int nsub, const void* x, const void* pe, const void* w1,
                            void* arows, float* y, float* pe_part, hipStream_t s) {
  const int R = dm.l / dm.d, KK = dm.d * D, H = dm.hidden;
  const size_t M = (size_t)dm.B * dm.Hkv * nsub + R;
  const size_t total = M * (KK / 8);
  const bool bf = dm.io == IO_BF16;
  if (bf)
    k_phi_arows<bf16><<<(unsigned)((total + 255) / 256), 256, 0, s>>>(dm, D, nsub, (const bf16*)x, (const bf16*)pe,
                                                                       (bf16*)arows);
  else
    k_phi_arows<float><<<(unsigned)((total + 255) / 256), 256, 0, s>>>(dm, D, nsub, (const float*)x,
                                                                        (const float*)pe, (float*)arows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the position-embedding rows, then the sub-block rows:
  // y[:, r*H : (r+1)*H] = A * w1[r*KK : (r+1)*KK, :], with bf16 I/O one
  // launch over the R chunks
  const size_t Mmain = M - R;
  {
    const dim3 grid((H + 63) / 64, R, kPeSlices);
    if (bf)
      k_phi_pe_part<bf16><<<grid, 256, 0, s>>>(dm, D, (const bf16*)pe, (const bf16*)w1, pe_part);
    else
      k_phi_pe_part<float><<<grid, 256, 0, s>>>(dm, D, (const float*)pe, (const float*)w1, pe_part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_phi_pe_fin<<<(R * H + 255) / 256, 256, 0, s>>>(dm, Mmain, pe_part, y);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const size_t es = bf ? 2 : 4;
  if (bf) {
    MmArgs g{(int)Mmain, H, KK, arows, KK, 1, w1, H, 1, y, R * H, 0, 0};
    g.batch = R;
    g.bsb = (long long)KK * H;
    g.bsc = H;
    return mm(g, false, false, 1, nullptr, s);
  }
  for (int r = 0; r < R; ++r) {
    const void* br = (const char*)w1 + (size_t)r * KK * H * es;
    {
      const Gemm g{(int)Mmain, H, KK, arows, KK, 1, br, H, 1, y + (size_t)r * H, R * H, 0};
      e = gemm_exact(g, true, true, nullptr, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_phi_mlp(const Dims& dm, const PhiMlpArgs& a, hipStream_t s) {
  if (dm.ncmp == 0) return hipSuccess;
  const bool bf = dm.io == IO_BF16;
  switch (a.D) {
    case 64: return bf ? phi_mlp_impl<bf16, 64>(dm, a, s) : phi_mlp_impl<float, 64>(dm, a, s);
    case 128: return bf ? phi_mlp_impl<bf16, 128>(dm, a, s) : phi_mlp_impl<float, 128>(dm, a, s);
    case 192: return bf ? phi_mlp_impl<bf16, 192>(dm, a, s) : phi_mlp_impl<float, 192>(dm, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nsa
