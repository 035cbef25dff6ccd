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
// Element e of a fragment in its own type, and a store of four such elements
// as one 8-byte (bf16) or 16-byte (fp32) vector.
__device__ __forceinline__ bf16 frag_at(const Frag8<bf16>& f, int e) { return f.v[e]; }
__device__ __forceinline__ float frag_at(const Frag8<float>& f, int e) { return e < 4 ? f.lo[e] : f.hi[e - 4]; }
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_col4(bf16* p, bf16 a, bf16 b, bf16 c, bf16 d) {
  *reinterpret_cast<bf16x4v*>(p) = bf16x4v{a, b, c, d};
}
__device__ __forceinline__ void store_col4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Transposed store of a 4-row x 8-element block: element e of rows 0..3 goes
// to dst[e * stride + 0..3].  The bf16 form pairs half-words with byte
// permutes, so no element is extracted through memory.
__device__ __forceinline__ void store_cols4x8(bf16* dst, int stride, const Frag8<bf16> (&r)[4]) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
  u32x4v w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = __builtin_bit_cast(u32x4v, r[k].v);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const unsigned lo01 = __builtin_amdgcn_perm(w[1][m], w[0][m], 0x05040100u);
    const unsigned lo23 = __builtin_amdgcn_perm(w[3][m], w[2][m], 0x05040100u);
    const unsigned hi01 = __builtin_amdgcn_perm(w[1][m], w[0][m], 0x07060302u);
    const unsigned hi23 = __builtin_amdgcn_perm(w[3][m], w[2][m], 0x07060302u);
    *reinterpret_cast<u32x2v*>(dst + (2 * m) * stride) = u32x2v{lo01, lo23};
    *reinterpret_cast<u32x2v*>(dst + (2 * m + 1) * stride) = u32x2v{hi01, hi23};
  }
}
__device__ __forceinline__ void store_cols4x8(float* dst, int stride, const Frag8<float> (&r)[4]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    store_col4(dst + e * stride, frag_at(r[0], e), frag_at(r[1], e), frag_at(r[2], e), frag_at(r[3], e));
}

// Streaming variants: data read or written once per kernel (query rows,
// outputs) carry the non-temporal hint so they do not displace reused data
// (key/value tiles) from L2 and the MALL.
__device__ __forceinline__ Frag8<bf16> load_frag_nt(const bf16* p) {
  Frag8<bf16> f;
  f.v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
  return f;
}
__device__ __forceinline__ Frag8<float> load_frag_nt(const float* p) {
  Frag8<float> f;
  f.lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  f.hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
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

// Two fp32 values -> two bf16 (round to nearest even) in one packed convert.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x2v cvt2_bf16(float a, float b) {
  return __builtin_convertvector((f32x2v){a, b}, bf16x2v);
}

// 8 fp32 values -> operand fragment of element type T (round to nearest even).
__device__ __forceinline__ Frag8<bf16> to_frag_bf16(const float* x) {
  Frag8<bf16> f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2v h = cvt2_bf16(x[e], x[e + 1]);
    f.v[e] = h[0];
    f.v[e + 1] = h[1];
  }
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
// Pairs are converted together and hi is widened back to fp32 by bit shifts.
__device__ __forceinline__ void split_bf16(const float* x, Frag8<bf16>& hi, Frag8<bf16>& lo) {
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2v h = cvt2_bf16(x[e], x[e + 1]);
    const unsigned hb = __builtin_bit_cast(unsigned, h);
    const bf16x2v l = cvt2_bf16(x[e] - __uint_as_float(hb << 16), x[e + 1] - __uint_as_float(hb & 0xffff0000u));
    hi.v[e] = h[0];
    hi.v[e + 1] = h[1];
    lo.v[e] = l[0];
    lo.v[e + 1] = l[1];
  }
}

// Residual of rounding x to the bf16 fragment hi: lo = bf16(x - hi), so that
// hi + lo carries ~16 significant bits of x.
__device__ __forceinline__ Frag8<bf16> lo_frag(const float* x, const Frag8<bf16>& hi) {
  Frag8<bf16> lo;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2v l = cvt2_bf16(x[e] - (float)hi.v[e], x[e + 1] - (float)hi.v[e + 1]);
    lo.v[e] = l[0];
    lo.v[e + 1] = l[1];
  }
  return lo;
}
__device__ __forceinline__ Frag8<float> lo_frag(const float*, const Frag8<float>&) { return Frag8<float>{}; }

// Attention outputs kept in fp32 for the backward (OT = float) with bf16
// inputs: P enters the P V product as hi + lo bf16 parts, so the saved branch
// outputs carry P to ~16 bits instead of 8.
template <typename T, typename OT>
constexpr bool kPrecisePV = sizeof(T) == 2 && sizeof(OT) == 4;

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
__device__ __forceinline__ void store4_nt(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
  __builtin_nontemporal_store(v, reinterpret_cast<bf16x4*>(p));
}
__device__ __forceinline__ void store4_nt(float* p, float a, float b, float c, float d) {
  __builtin_nontemporal_store(f32x4{a, b, c, d}, reinterpret_cast<f32x4*>(p));
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

// Selected-block rows (n entries per position and KV head, ascending, -1
// padded) are read in order while each entry is above the previous one (the
// first above -1) and causal (its first token j*ls <= t).  Every kernel that
// reads a row caller-side (the backward takes the forward's rows back from the
// caller) applies this rule, so entries after padding, a repeated or
// descending entry, or a block past t are never used to address memory, and
// all kernels use the same entries.
__host__ __device__ __forceinline__ bool sel_slot_ok(int j, int prev, int t, int ls) {
  return j > prev && j >= 0 && j <= t / ls;
}

// Length of the usable prefix of a row whose entry si sits in lane si (-1 in
// lanes si >= n); one wave, every lane gets the same count.
__device__ __forceinline__ int wave_sel_row_len(int myid, int lane, int n, int t, int ls) {
  const int prev = __shfl_up(myid, 1);
  const bool bad = lane < n && !sel_slot_ok(myid, lane == 0 ? -1 : prev, t, ls);
  const uint64_t stop = __ballot(bad || lane >= n);
  return stop ? __builtin_ctzll(stop) : 64;
}

// ---------------------------------------------------------------------------
// Workgroup -> (batch*kv-head unit, tile) mapping.  Workgroups are handed to
// the 8 XCDs round-robin by id; this keeps every XCD on one (batch, kv head)
// unit when there are at most 8 units (so that unit's keys stay in that
// XCD's L2), and hands out the most expensive tiles (late positions) first.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ void xcd_map(int id, int units, int ntiles, int& unit, int& tile) {
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

// Output tile (row tile mt, column tile nt) of GEMM workgroup lid in an
// ncol x nrow grid.  Workgroups are dispatched to the 8 XCDs in turn: with a
// multiple of 8 row tiles, XCD x takes row tiles x, x+8, ... and each one's
// column tiles back to back, so the A rows of a row tile are fetched into one
// L2 while its column tiles run; otherwise tiles go in launch order.
__host__ __device__ __forceinline__ void gemm_tile_order(int lid, int ncol, int nrow, int& mt, int& nt) {
  if (nrow % 8 == 0) {
    const int x = lid & 7, k = lid >> 3;
    mt = (k / ncol) * 8 + x;
    nt = k % ncol;
  } else {
    mt = lid / ncol;
    nt = lid % ncol;
  }
}

// A GEMM whose n range is cut into nseg segments (segment s holds columns
// [off[s], off[s + 1]), the last one ending at N), each padded to whole tiles
// of tw columns, so that no tile spans two segments.  seg_tiles: the column
// tile count; seg_tile: segment s of column tile nt and that tile's first
// column inside the segment.
__host__ __device__ __forceinline__ int seg_width(int s, int nseg, const int* off, int N) {
  return (s + 1 < nseg ? off[s + 1] : N) - off[s];
}
__host__ __device__ __forceinline__ int seg_tiles(int nseg, const int* off, int N, int tw) {
  int t = 0;
  for (int s = 0; s < nseg; ++s) t += (seg_width(s, nseg, off, N) + tw - 1) / tw;
  return t;
}
__host__ __device__ __forceinline__ void seg_tile(int nt, int nseg, const int* off, int N, int tw, int& s, int& n0) {
  int t0 = 0;
  for (s = 0; s + 1 < nseg; ++s) {
    const int tc = (seg_width(s, nseg, off, N) + tw - 1) / tw;
    if (nt < t0 + tc) break;
    t0 += tc;
  }
  n0 = (nt - t0) * tw;
}

// Task (group kg, segment seg) of workgroup id, for units x ngroup x nseg
// tasks whose query rows start at kg*span + seg*seglen (plus a constant).
// When span is a multiple of seglen, the tasks with equal a = R*kg + seg
// (R = span / seglen) read the same rows: each XCD then takes one unit's
// tasks in increasing a (xcd_map), so the tasks running together on it share
// their rows in L2.  Otherwise the unit index runs fastest.  A bijection of
// [0, units*ngroup*nseg) onto the tasks either way.
__host__ __device__ __forceinline__ void span_task_order(int id, int units, int ngroup, int nseg, int span,
                                                         int seglen, int& unit, int& kg, int& seg) {
  if (span % seglen == 0) {
    const int R = span / seglen;
    int tile;
    xcd_map(id, units, ngroup * nseg, unit, tile);
    int r = ngroup * nseg - 1 - tile;   // rank among the unit's tasks
    const int amax = R * (ngroup - 1) + nseg - 1;
    for (int a = 0; a <= amax; ++a) {
      // groups kg < ngroup with 0 <= a - R*kg < nseg
      const int hi = a / R < ngroup - 1 ? a / R : ngroup - 1;
      const int lo = a - nseg + 1 <= 0 ? 0 : (a - nseg + R) / R;
      const int cnt = hi >= lo ? hi - lo + 1 : 0;
      if (r < cnt) {
        kg = lo + r;
        seg = a - R * kg;
        return;
      }
      r -= cnt;
    }
  }
  unit = id % units;
  const int r = id / units;
  kg = r % ngroup;
  seg = r / ngroup;
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

// Wave-wide max (float) and min (int) by the same DPP pattern, broadcast.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_f32(float v, float ident) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(ident), __float_as_int(v), CTRL, ROWMASK, 0xf,
                                                    false));
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_i32(int v, int ident) {
  return __builtin_amdgcn_update_dpp(ident, v, CTRL, ROWMASK, 0xf, false);
}
__device__ __forceinline__ float wave_max_f32(float v) {
  const float ni = -__builtin_inff();
  v = fmaxf(v, dpp_f32<0x111, 0xf>(v, ni));
  v = fmaxf(v, dpp_f32<0x112, 0xf>(v, ni));
  v = fmaxf(v, dpp_f32<0x114, 0xf>(v, ni));
  v = fmaxf(v, dpp_f32<0x118, 0xf>(v, ni));
  v = fmaxf(v, dpp_f32<0x142, 0xa>(v, ni));
  v = fmaxf(v, dpp_f32<0x143, 0xc>(v, ni));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int wave_min_i32(int v) {
  const int id = 0x7fffffff;
  v = min(v, dpp_i32<0x111, 0xf>(v, id));
  v = min(v, dpp_i32<0x112, 0xf>(v, id));
  v = min(v, dpp_i32<0x114, 0xf>(v, id));
  v = min(v, dpp_i32<0x118, 0xf>(v, id));
  v = min(v, dpp_i32<0x142, 0xa>(v, id));
  v = min(v, dpp_i32<0x143, 0xc>(v, id));
  return __builtin_amdgcn_readlane(v, 63);
}
// Wave-wide maximum of an unsigned value (0 is the identity), broadcast.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i32<0x111, 0xf>((int)v, 0));
  v = max(v, (uint32_t)dpp_i32<0x112, 0xf>((int)v, 0));
  v = max(v, (uint32_t)dpp_i32<0x114, 0xf>((int)v, 0));
  v = max(v, (uint32_t)dpp_i32<0x118, 0xf>((int)v, 0));
  v = max(v, (uint32_t)dpp_i32<0x142, 0xa>((int)v, 0));
  v = max(v, (uint32_t)dpp_i32<0x143, 0xc>((int)v, 0));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Selection order: larger score first, the lower index winning a tie.  Each
// lane offers its best (s, j); the wave's best is returned in every lane
// (s = -inf when no lane has a candidate).
__device__ __forceinline__ void wave_argmax(float s, int j, float& bs, int& bj) {
  bs = wave_max_f32(s);
  bj = wave_min_i32(s == bs ? j : 0x7fffffff);
}
__device__ __forceinline__ bool topn_better(float s, int j, float bs, int bj) {
  return s > bs || (s == bs && j < bj);
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
  // each lane keeps its best candidate among j = lane (mod 64)
  float ms;
  int mj;
  auto lane_best = [&]() {
    ms = -__builtin_inff();
    mj = 0x7fffffff;
    for (int j = lane; j <= jc; j += 64) {
      const float v = row[j];
      if (v >= 0.f && v > ms) { ms = v; mj = j; }
    }
  };
  lane_best();
  for (int it = 0; it < n - 3; ++it) {
    float bs;
    int bj;
    wave_argmax(ms, mj, bs, bj);
    if (bs < 0.f) break;
    if (mj == bj) {
      row[bj] = -1.f;
      lane_best();
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

// The same selection for R rows at once, each held in registers (rows of at
// most 64*KV blocks): lane L owns blocks L + 64 i (i < KV), read from LDS
// once, as 32-bit keys: the score's bits plus one (scores are >= 0, so their
// bits order like their values; 0 marks a block that is not a candidate).
// Each lane keeps its three best unselected keys with their slots i, sorted
// by key and, among equal keys, by lower slot (a lane's blocks ascend with i).
// A pick is one 32-bit wave maximum per row (the R chains are independent);
// the lanes holding it are found by ballot, and when several lanes hold equal
// keys the lowest block index among them wins, as in the selection rule.  The
// winning lane shifts its three keys and re-ranks its blocks only when all
// three were taken.  t[r] < 0 marks an absent row.
template <int KV, int R>
__device__ inline void wave_topn_rows(const float* const* row, const int* t, int ls, int n, int* const* out,
                                      int lane) {
  int jc[R];
  bool live[R];
  uint32_t key[R][KV];
  uint32_t taken[R];     // bit i: block lane + 64 i selected
  uint32_t k1[R], k2[R], k3[R];
  int i1[R], i2[R], i3[R];
  auto rank3 = [&](int r) {
    uint32_t a = 0, b = 0, c = 0;
    int ia = 0, ib = 0, ic = 0;
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const uint32_t x = (taken[r] >> i) & 1u ? 0u : key[r][i];
      // strict: of two equal keys the one met first (lower block) stays ahead
      const bool g1 = x > a, g2 = x > b, g3 = x > c;
      c = g2 ? b : (g3 ? x : c);
      ic = g2 ? ib : (g3 ? i : ic);
      b = g1 ? a : (g2 ? x : b);
      ib = g1 ? ia : (g2 ? i : ib);
      a = g1 ? x : a;
      ia = g1 ? i : ia;
    }
    k1[r] = a;
    k2[r] = b;
    k3[r] = c;
    i1[r] = ia;
    i2[r] = ib;
    i3[r] = ic;
  };
#pragma unroll
  for (int r = 0; r < R; ++r) {
    jc[r] = t[r] >= 0 ? t[r] / ls : -1;
    live[r] = t[r] >= 0 && jc[r] + 1 > n;
    taken[r] = 0;
    if (t[r] >= 0 && !live[r])
      for (int e = lane; e < n; e += 64) out[r][e] = e <= jc[r] ? e : -1;
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int j = lane + 64 * i;
      const bool cand = live[r] && j <= jc[r] && j != 0 && j != jc[r] - 1 && j != jc[r];
      key[r][i] = cand ? (__float_as_uint(row[r][j]) & 0x7fffffffu) + 1u : 0u;
    }
    rank3(r);
  }
  for (int it = 0; it < n - 3; ++it) {
    uint32_t best[R];
#pragma unroll
    for (int r = 0; r < R; ++r) best[r] = wave_max_u32(k1[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (best[r] == 0u) continue;   // no candidate left in this row
      const uint64_t holders = __ballot(k1[r] == best[r]);
      int win;
      if (__popcll(holders) == 1) {
        win = __builtin_ctzll(holders);
      } else {
        // equal keys in several lanes: the lowest block index j = lane + 64 i
        win = wave_min_i32(k1[r] == best[r] ? lane + 64 * i1[r] : 0x7fffffff) & 63;
      }
      if (lane == win) {
        taken[r] |= 1u << i1[r];
        k1[r] = k2[r];
        i1[r] = i2[r];
        k2[r] = k3[r];
        i2[r] = i3[r];
        k3[r] = 0u;
        if (k1[r] == 0u) rank3(r);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!live[r]) continue;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      if (64 * i > jc[r]) break;
      const int j = lane + 64 * i;
      const bool sel = j <= jc[r] && (((taken[r] >> i) & 1u) || j == 0 || j == jc[r] - 1 || j == jc[r]);
      const uint64_t mk = __ballot(sel);
      if (sel) out[r][cnt + __popcll(mk & ((1ull << lane) - 1ull))] = j;
      cnt += __popcll(mk);
    }
    for (int e = cnt + lane; e < n; e += 64) out[r][e] = -1;
  }
}

// The same selection by a whole workgroup of NW waves (NW*64 threads), by
// radix select instead of repeated argmax.  Scores are >= 0, so their bit
// patterns order like the values.  Four passes over 8-bit digits, most
// significant first, narrow down the bit pattern K of the r-th largest
// non-forced score (r = n - 3) and how many of the scores equal to K are still
// needed; those are the lowest-indexed ones (ties go to the lower index).  The
// selected set, forced blocks included, is then written in ascending order.
// sh: LDS scratch of 256 + NW + 4 ints.  The caller synchronises the workgroup
// before (row complete) and after.
template <int NW>
__device__ inline void block_topn(const float* row, int t, int ls, int n, int* out, int* sh, int tid) {
  constexpr int NT = NW * 64;
  const int jc = t / ls;
  if (jc + 1 <= n) {
    for (int e = tid; e < n; e += NT) out[e] = e <= jc ? e : -1;
    return;
  }
  const int lane = tid & 63, wave = tid >> 6;
  int* hist = sh;              // [256]
  int* wcnt = sh + 256;        // [NW] per-wave counts
  int* ctl = wcnt + NW;        // [0] digit prefix, [1] still needed, [2] running total
  auto key = [&](int j) { return __float_as_uint(row[j]); };
  auto forced = [&](int j) { return j == 0 || j == jc - 1 || j == jc; };
  unsigned prefix = 0, mask = 0;
  int need = n - 3;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j <= jc; j += NT) {
      if (forced(j)) continue;
      const unsigned u = key(j);
      if ((u & mask) == prefix) atomicAdd(hist + ((u >> shift) & 255), 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane L holds bins 255-4L .. 252-4L; counts are summed from the top
      int h[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { h[i] = hist[255 - 4 * lane - i]; sum += h[i]; }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      int run = incl - sum;   // bins above this lane's
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (run < need && run + h[i] >= need) {
          ctl[0] = 255 - 4 * lane - i;
          ctl[1] = need - run;
        }
        run += h[i];
      }
    }
    __syncthreads();
    prefix |= (unsigned)ctl[0] << shift;
    mask |= 255u << shift;
    need = ctl[1];
    __syncthreads();
  }
  // Selection in index order: a score above K, or equal to K among the first
  // `need` such indices, or a forced block.  Two workgroup prefix counts (over
  // 'equal to K', then over 'selected') walk the candidates in chunks of NT.
  if (tid == 0) { ctl[1] = 0; ctl[2] = 0; }
  __syncthreads();
  for (int j0 = 0; j0 <= jc; j0 += NT) {
    const int j = j0 + tid;
    const bool valid = j <= jc;
    const unsigned u = valid ? key(j) : 0u;
    const bool eq = valid && !forced(j) && u == prefix;
    // rank of j among the equal scores
    uint64_t bal = __ballot(eq);
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    int before = ctl[1];
    for (int w = 0; w < wave; ++w) before += wcnt[w];
    const int rank = before + __popcll(bal & ((1ull << lane) - 1ull));
    const bool sel = valid && (forced(j) || u > prefix || (eq && rank < need));
    __syncthreads();
    if (tid == NT - 1) {
      int tot = ctl[1];
      for (int w = 0; w < NW; ++w) tot += wcnt[w];
      ctl[1] = tot;
    }
    // position of j among the selected blocks
    bal = __ballot(sel);
    __syncthreads();
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    int pos = ctl[2];
    for (int w = 0; w < wave; ++w) pos += wcnt[w];
    pos += __popcll(bal & ((1ull << lane) - 1ull));
    if (sel && pos < n) out[pos] = j;
    __syncthreads();
    if (tid == NT - 1) {
      int tot = ctl[2];
      for (int w = 0; w < NW; ++w) tot += wcnt[w];
      ctl[2] = tot;
    }
    __syncthreads();
  }
  const int cnt = ctl[2];
  for (int e = cnt + tid; e < n; e += NT) out[e] = -1;
}

}  // namespace nsa
