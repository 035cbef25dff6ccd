// Device helpers shared by the gfx950 NSA kernels: MFMA fragments, conversions,
// wave reductions and the workgroup -> XCD work mapping.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// One lane's share of an MFMA operand: 8 consecutive elements along the
// contraction index.  For v_mfma_f32_16x16x32_bf16 lane l holds row (or
// column) l%16 and contraction indices 8*(l/16) .. 8*(l/16)+7.  The fp32
// variant issues eight v_mfma_f32_16x16x4_f32, the e-th contracting element e
// of every lane, which sums the same 32 products.
// ---------------------------------------------------------------------------
template <typename T> struct Frag8;
template <> struct Frag8<bf16> { bf16x8 v; };
template <> struct Frag8<float> { f32x4 lo, hi; };

__device__ __forceinline__ Frag8<bf16> load_frag(const bf16* p) {
  Frag8<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag8<float> load_frag(const float* p) {
  Frag8<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f;
}
template <typename T> __device__ __forceinline__ Frag8<T> zero_frag();
template <> __device__ __forceinline__ Frag8<bf16> zero_frag<bf16>() {
  Frag8<bf16> f;
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)0.0f;
  return f;
}
template <> __device__ __forceinline__ Frag8<float> zero_frag<float>() {
  Frag8<float> f;
  for (int e = 0; e < 4; ++e) { f.lo[e] = 0.f; f.hi[e] = 0.f; }
  return f;
}

__device__ __forceinline__ void mma(f32x4& c, const Frag8<bf16>& a, const Frag8<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const Frag8<float>& a, const Frag8<float>& b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[e], b.lo[e], c, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[e], b.hi[e], c, 0, 0, 0);
}

// 8 fp32 values -> operand fragment of element type T (round to nearest even).
__device__ __forceinline__ Frag8<bf16> to_frag_bf16(const float* x) {
  Frag8<bf16> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)x[e];
  return f;
}
template <typename T> __device__ __forceinline__ Frag8<T> to_frag(const float* x);
template <> __device__ __forceinline__ Frag8<bf16> to_frag<bf16>(const float* x) { return to_frag_bf16(x); }
template <> __device__ __forceinline__ Frag8<float> to_frag<float>(const float* x) {
  Frag8<float> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.lo[e] = x[e]; f.hi[e] = x[4 + e]; }
  return f;
}
// x = hi + lo with hi, lo in bf16: the pair carries ~16 significant bits.
__device__ __forceinline__ void split_bf16(const float* x, Frag8<bf16>& hi, Frag8<bf16>& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16 h = (bf16)x[e];
    hi.v[e] = h;
    lo.v[e] = (bf16)(x[e] - (float)h);
  }
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

// Store 4 consecutive values.
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  f32x4 v;
  v[0] = a; v[1] = b; v[2] = c; v[3] = d;
  *reinterpret_cast<f32x4*>(p) = v;
}
__device__ __forceinline__ void load4(const bf16* p, float* o) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  o[0] = (float)v[0]; o[1] = (float)v[1]; o[2] = (float)v[2]; o[3] = (float)v[3];
}
__device__ __forceinline__ void load4(const float* p, float* o) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Number of complete compression blocks [i*d, i*d+l) whose last token is <= t.
__device__ __forceinline__ int ncmp_visible(int t, int l, int d) {
  int s = t + 1;
  return s < l ? 0 : (s - l) / d + 1;
}

// ---------------------------------------------------------------------------
// Workgroup -> (batch*kv-head unit, tile) mapping.  Workgroups are handed to
// the 8 XCDs round-robin by id; this keeps every XCD on one (batch, kv head)
// unit when there are at most 8 units (so that unit's keys stay in that
// XCD's L2), and hands out the most expensive tiles (late positions) first.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void xcd_map(int id, int units, int ntiles, int& unit, int& tile) {
  if (units <= 8 && 8 % units == 0 && ntiles % (8 / units) == 0) {
    int per = 8 / units, x = id & 7, k = id >> 3;
    unit = x / per;
    tile = ntiles - 1 - (k * per + x % per);
  } else if (units % 8 == 0) {
    int x = id & 7, k = id >> 3;
    unit = x + 8 * (k / ntiles);
    tile = ntiles - 1 - k % ntiles;
  } else {
    unit = id / ntiles;
    tile = ntiles - 1 - id % ntiles;
  }
}

// Weight of compression block kr (row of a 32-key tile) in selection block jc
// (column of the tile's window), in units of d: the overlap of their token
// ranges [kr*d, kr*d+l) and [jc*ls, (jc+1)*ls), divided by d.
__device__ __forceinline__ float remap_weight(int kr, int jc, int l, int d, int ls) {
  const int a0 = kr * d, a1 = a0 + l, b0 = jc * ls, b1 = b0 + ls;
  const int ov = min(a1, b1) - max(a0, b0);
  return ov > 0 ? (float)(ov / d) : 0.f;
}

// ---------------------------------------------------------------------------
// Cross-lane exchanges without the LDS crossbar (gfx950 permlane swaps, DPP).
// xor16 / xor32 return the value of lane ^ 16 / lane ^ 32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor16f(float v, int lane) {
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((lane & 16) ? q[0] : q[1]);
}
__device__ __forceinline__ float xor32f(float v, int lane) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((lane & 32) ? p[0] : p[1]);
}
// Reductions over the 4 lanes that share lane % 16 (one MFMA column).
__device__ __forceinline__ float colmax4(float v, int lane) {
  v = fmaxf(v, xor16f(v, lane));
  return fmaxf(v, xor32f(v, lane));
}
__device__ __forceinline__ float colsum4(float v, int lane) {
  v += xor16f(v, lane);
  return v + xor32f(v, lane);
}

template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWMASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWMASK, 0xf, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
// Maximum of a 64-bit key over the wave (DPP prefix max ends in lane 63), broadcast.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  uint64_t t;
  t = dpp_u64<0x111, 0xf>(k); k = t > k ? t : k;   // row_shr:1
  t = dpp_u64<0x112, 0xf>(k); k = t > k ? t : k;   // row_shr:2
  t = dpp_u64<0x114, 0xf>(k); k = t > k ? t : k;   // row_shr:4
  t = dpp_u64<0x118, 0xf>(k); k = t > k ? t : k;   // row_shr:8
  t = dpp_u64<0x142, 0xa>(k); k = t > k ? t : k;   // row_bcast:15
  t = dpp_u64<0x143, 0xc>(k); k = t > k ? t : k;   // row_bcast:31
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)k, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}
// Order key of candidate block j with score v >= 0: larger score first, then
// lower index.  Taken (marked, v < 0) entries map to 0, below every candidate.
__device__ __forceinline__ uint64_t topn_key(float v, int j) {
  return v < 0.f ? 0ull : ((uint64_t)__float_as_uint(v) << 32) | (uint32_t)(0xffffffffu - (uint32_t)j);
}

// Top-n block selection for query position t from one group's score row
// (LDS, nsel entries, scores >= 0), executed by one whole wave.  Block 0 and
// blocks floor(t/ls) and floor(t/ls)-1 are always selected; the remaining
// n-3 slots go to the highest scores among the other causal blocks
// j <= floor(t/ls), the lower index winning a tie.  When at most n blocks
// are causal all are selected.  Writes n indices ascending, -1 padded.  The
// row is overwritten (selected entries marked -1).
__device__ inline void wave_topn(float* row, int t, int ls, int n, int* out, int lane) {
  const int jc = t / ls;
  if (jc + 1 <= n) {
    for (int e = lane; e < n; e += 64) out[e] = e <= jc ? e : -1;
    return;
  }
  if (lane == 0) { row[0] = -1.f; row[jc - 1] = -1.f; row[jc] = -1.f; }
  // each lane keeps the best key among its candidates j = lane (mod 64)
  auto lane_best = [&]() {
    uint64_t best = 0;
    for (int j = lane; j <= jc; j += 64) {
      const uint64_t k = topn_key(row[j], j);
      best = k > best ? k : best;
    }
    return best;
  };
  uint64_t mine = lane_best();
  for (int it = 0; it < n - 3; ++it) {
    const uint64_t win = wave_max_u64(mine);
    const int bj = (int)(0xffffffffu - (uint32_t)win);
    if ((bj & 63) == lane) {
      row[bj] = -1.f;
      mine = lane_best();
    }
  }
  int cnt = 0;
  for (int jb = 0; jb <= jc; jb += 64) {
    const int j = jb + lane;
    const bool sel = j <= jc && row[j] < 0.f;
    const uint64_t mk = __ballot(sel);
    if (sel) out[cnt + __popcll(mk & ((1ull << lane) - 1ull))] = j;
    cnt += __popcll(mk);
  }
  for (int e = cnt + lane; e < n; e += 64) out[e] = -1;
}

}  // namespace nsa
