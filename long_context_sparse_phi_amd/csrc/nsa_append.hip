// Decode-time cache maintenance for gfx950: one new token per sequence goes
// into the raw key/value caches, and the compression block it completes, if
// any, is compressed into the next row of the compressed caches.
//
// youleyou NSA page, 令牌压缩: block i covers tokens [i*d, i*d+l); phi maps it
// to one compressed key (value).  During decoding a block becomes available
// when its last token arrives, i.e. when the sequence length L+1 satisfies
// L+1 >= l and (L+1-l) % d == 0; it is then block (L+1-l)/d.
//
// Work per call is tiny (at most one block per (sequence, KV head)) and bound
// by latency: the MLP phi's first layer runs as a 16-row MFMA GEMM over the
// l*D block features of the rows that complete a block, split over the
// feature axis into 256-wide slices so that hundreds of workgroups each do a
// few steps (W1 column tiles staged through LDS); the second kernel sums the
// slices, applies the GELU and evaluates the second layer in fp32 with one
// thread per output feature.  Rows that do not complete a block skip all work.
#include "nsa_common.hpp"
#include "nsa_kernels.hpp"

namespace nsa {

// Cache slot of sequence b's new token, or -1 when the cache is full (or the
// stored length is negative).
__device__ __forceinline__ int append_slot(const int* lens, int b, int S) {
  const int L = lens[b];
  return (L >= 0 && L < S) ? L : -1;
}

// Compression block completed by a token at slot L, or -1.
__device__ __forceinline__ int append_block(int L, int l, int d) {
  if (L < 0) return -1;
  const int n = L + 1 - l;
  return (n >= 0 && n % d == 0) ? n / d : -1;
}

// Raw caches: k_cache[b, L, g] = k_new[b, g] and the same for v, for the
// compressed branch's pair (blockIdx.y = 0) and, when given, the selected
// (1) and window (2) branches' own pairs.
template <typename T>
__global__ __launch_bounds__(64) void k_append_store(Dims dm, AppendArgs a) {
  const int bg = blockIdx.x, b = bg / dm.Hkv, g = bg % dm.Hkv;
  const T* kn = (const T*)(blockIdx.y == 0 ? a.kn : blockIdx.y == 1 ? a.kn_slc : a.kn_win);
  const T* vn = (const T*)(blockIdx.y == 0 ? a.vn : blockIdx.y == 1 ? a.vn_slc : a.vn_win);
  T* kc = (T*)(blockIdx.y == 0 ? a.kc : blockIdx.y == 1 ? a.kc_slc : a.kc_win);
  T* vc = (T*)(blockIdx.y == 0 ? a.vc : blockIdx.y == 1 ? a.vc_slc : a.vc_win);
  const int L = append_slot(a.lens, b, dm.T);
  if (L < 0 || !kc) return;
  const size_t rk = (size_t)(b * dm.T + L) * dm.Hkv + g;
  for (int e = threadIdx.x; e < dm.dk; e += 64) kc[rk * dm.dk + e] = kn[(size_t)bg * dm.dk + e];
  for (int e = threadIdx.x; e < dm.dv; e += 64) vc[rk * dm.dv + e] = vn[(size_t)bg * dm.dv + e];
}

// Mean-pool phi of the completed block: (1/l) sum_j x[i*d + j], summed in
// token order in fp32.
template <typename T>
__global__ __launch_bounds__(64) void k_append_mean(Dims dm, int D, int cap, const int* __restrict__ lens,
                                                    const T* __restrict__ x, T* __restrict__ out) {
  const int bg = blockIdx.x, b = bg / dm.Hkv, g = bg % dm.Hkv;
  const int i = append_block(append_slot(lens, b, dm.T), dm.l, dm.d);
  if (i < 0) return;
  const T* src = x + ((size_t)(b * dm.T + i * dm.d) * dm.Hkv + g) * D;
  T* dst = out + ((size_t)(b * cap + i) * dm.Hkv + g) * D;
  for (int e = threadIdx.x; e < D; e += 64) {
    float acc = 0.f;
    for (int j = 0; j < dm.l; ++j) acc += to_f32(src[(size_t)j * dm.Hkv * D + e]);
    dst[e] = from_f32<T>(acc / (float)dm.l);
  }
}

constexpr int kAppendKS = 256;   // first-layer features per workgroup (split-K slice)

// MLP phi, first layer, one feature slice: part[z, r, n] = sum over x in slice z
// of u_r[x] w1[x, n] for the rows r = (b, g) that complete a block,
// u_r = concat_j (x[i*d+j] + pe[j]).  The pe term is a second MFMA on the
// same W1 fragment, so both operands stay exact in the I/O type.  Workgroup:
// 16 rows x 64 hidden units x one slice, one wave per 16 units;
// W1[kk .. kk+31][n0 .. n0+63] is staged transposed in LDS, the next step's
// global loads are issued before the current step's MFMAs.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_append_h(Dims dm, const int* __restrict__ lens, const T* __restrict__ x,
                                                  const T* __restrict__ pe, const T* __restrict__ w1,
                                                  float* __restrict__ part) {
  constexpr int WS = 32 + 8;              // LDS row stride (elements) of the transposed W1 tile
  __shared__ __align__(16) T ws[64 * WS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, qd = lane >> 4;
  const int R = dm.B * dm.Hkv, H = dm.hidden;
  const int r = blockIdx.y * 16 + c16;
  const int n0 = blockIdx.x * 64;
  const T* src = nullptr;
  if (r < R) {
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    const int i = append_block(append_slot(lens, b, dm.T), dm.l, dm.d);
    if (i >= 0) src = x + ((size_t)(b * dm.T + i * dm.d) * dm.Hkv + g) * D;
  }
  if (!__syncthreads_or(src != nullptr)) return;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const int k0 = blockIdx.z * kAppendKS, k1 = min(k0 + kAppendKS, dm.l * D);
  const int lr = tid >> 3, lc = (tid & 7) * 8;   // loader: W1 row kk+lr, columns n0+lc .. +7
  auto gload = [&](int kk, Frag8<T>& f, Frag8<T>& a, Frag8<T>& ap) {
    f = load_frag(w1 + (size_t)(kk + lr) * H + n0 + lc);
    const int xx = kk + qd * 8, j = xx / D, e = xx % D;
    a = src ? load_frag(src + (size_t)j * dm.Hkv * D + e) : zero_frag<T>();
    ap = load_frag(pe + xx);
  };
  Frag8<T> f, a, ap;
  gload(k0, f, a, ap);
  for (int kk = k0; kk < k1; kk += 32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ws[(lc + e) * WS + lr] = frag_at(f, e);
    __syncthreads();
    const Frag8<T> ca = a, cp = ap;
    if (kk + 32 < k1) gload(kk + 32, f, a, ap);
    const Frag8<T> bw = *reinterpret_cast<const Frag8<T>*>(ws + (wave * 16 + c16) * WS + qd * 8);
    mma(acc, ca, bw);
    mma(acc, cp, bw);
    __syncthreads();
  }
  // acc[k]: row 4*qd + k of the tile, hidden unit n0 + 16*wave + c16
  const int n = n0 + wave * 16 + c16;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = blockIdx.y * 16 + qd * 4 + k;
    if (rr < R) part[((size_t)blockIdx.z * R + rr) * H + n] = acc[k];
  }
}

// MLP phi, second layer: a = b1 + the sum of the first layer's slices (in
// slice order), h = gelu(a), out[b, i, g, e] = b2[e] + sum_n h[n] w2[n, e],
// fp32, one thread per feature.
template <typename T>
__global__ __launch_bounds__(256) void k_append_o(Dims dm, int D, int cap, int nslice, const int* __restrict__ lens,
                                                  const float* __restrict__ part, const T* __restrict__ b1,
                                                  const T* __restrict__ w2, const T* __restrict__ b2,
                                                  T* __restrict__ out) {
  extern __shared__ float hs[];
  const int r = blockIdx.x, b = r / dm.Hkv, g = r % dm.Hkv;
  const int i = append_block(append_slot(lens, b, dm.T), dm.l, dm.d);
  if (i < 0) return;
  const int H = dm.hidden, R = dm.B * dm.Hkv;
  for (int n = threadIdx.x; n < H; n += blockDim.x) {
    float av = to_f32(b1[n]);
#pragma unroll 8
    for (int z = 0; z < nslice; ++z) av += part[((size_t)z * R + r) * H + n];
    hs[n] = 0.5f * av * (1.f + erff(av * 0.70710678118654752f));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < D; e += blockDim.x) {
    float acc = to_f32(b2[e]);
#pragma unroll 16
    for (int n = 0; n < H; ++n) acc = fmaf(hs[n], to_f32(w2[(size_t)n * D + e]), acc);
    out[((size_t)(b * cap + i) * dm.Hkv + g) * D + e] = from_f32<T>(acc);
  }
}

static int append_slices(const Dims& dm, int D) { return (dm.l * D + kAppendKS - 1) / kAppendKS; }

size_t append_ws_bytes(const Dims& dm) {
  const int D = dm.dk > dm.dv ? dm.dk : dm.dv;
  return dm.hidden ? (size_t)append_slices(dm, D) * dm.B * dm.Hkv * dm.hidden * sizeof(float) : 0;
}

template <typename T, int D>
static hipError_t append_phi(const Dims& dm, const AppendArgs& a, const T* x, const AppendPhi& w, T* out,
                             hipStream_t s) {
  const int R = dm.B * dm.Hkv;
  if (dm.hidden == 0) {
    k_append_mean<T><<<R, 64, 0, s>>>(dm, D, a.cap, a.lens, x, out);
    return hipGetLastError();
  }
  const int ns = append_slices(dm, D);
  dim3 grid(dm.hidden / 64, (R + 15) / 16, ns);
  k_append_h<T, D><<<grid, 256, 0, s>>>(dm, a.lens, x, (const T*)w.pe, (const T*)w.w1, a.h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_append_o<T><<<R, 256, dm.hidden * sizeof(float), s>>>(dm, D, a.cap, ns, a.lens, a.h, (const T*)w.b1,
                                                          (const T*)w.w2, (const T*)w.b2, out);
  return hipGetLastError();
}

template <typename T, int DK, int DV>
static hipError_t append_impl(const Dims& dm, const AppendArgs& a, hipStream_t s) {
  const unsigned pairs = a.kc_win ? 3 : (a.kc_slc ? 2 : 1);
  k_append_store<T><<<dim3(dm.B * dm.Hkv, pairs), 64, 0, s>>>(dm, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dm.ncmp == 0) return hipSuccess;   // no block can complete within the capacity
  if ((e = append_phi<T, DK>(dm, a, (const T*)a.kc, a.phi_k, (T*)a.kcmp, s)) != hipSuccess) return e;
  return append_phi<T, DV>(dm, a, (const T*)a.vc, a.phi_v, (T*)a.vcmp, s);
}

hipError_t launch_append(const Dims& dm, const AppendArgs& a, hipStream_t s) {
  const bool bf = dm.io == IO_BF16;
  if (dm.dk == 64 && dm.dv == 64) return bf ? append_impl<bf16, 64, 64>(dm, a, s) : append_impl<float, 64, 64>(dm, a, s);
  if (dm.dk == 128 && dm.dv == 128) return bf ? append_impl<bf16, 128, 128>(dm, a, s) : append_impl<float, 128, 128>(dm, a, s);
  if (dm.dk == 192 && dm.dv == 128) return bf ? append_impl<bf16, 192, 128>(dm, a, s) : append_impl<float, 192, 128>(dm, a, s);
  return hipErrorInvalidValue;
}

}  // namespace nsa
