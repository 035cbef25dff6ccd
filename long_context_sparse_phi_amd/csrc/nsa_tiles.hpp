// Cooperative staging of 64-key attention tiles in LDS for a workgroup of NT
// threads: a K tile [64 keys][DK] and a V^T tile [DV][64 keys].  Global loads
// go to registers first (gload) so they can be in flight while the previous
// tile is computed, then to LDS (lstore).
//
// K rows are unpadded; their 16-byte chunks are XOR-swizzled by row
// (kswz) so that the 16 key rows one MFMA fragment read touches land in 16
// different 4-bank groups.  The rows read together are the permuted key rows
// (c/4)*8 + c%4 (+4), c = 0..15; kswz is a bijection on the chunks of a row.
// bf16 V^T rows (128 bytes) are unpadded with chunk c of row r stored at
// c ^ ((r >> 1) & 7): measured on gfx950, the 16-row fragment reads and the
// 8-lanes-per-row stores of this layout are free of bank conflicts, while
// rows padded to 72 elements are not.  fp32 V^T rows stay padded.
#pragma once
#include "nsa_common.hpp"

namespace nsa {

constexpr int kTileKeys = 64;
constexpr int kTileVS = kTileKeys + 8;

// XOR pattern of K-tile row r.  With a row length of 128 elements (256 bytes)
// every row starts in the same bank group, so 16 distinct 4-bit patterns are
// needed; with 64 or 192 elements odd rows are offset by half the banks and a
// 3-bit pattern distinct within each row parity suffices (and stays inside
// aligned groups of 8 chunks).
template <int DK>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (DK == 128) return (r & 3) | ((r >> 3 & 3) << 2);
  else return (r >> 1 & 1) | (r >> 2 & 6);
}
template <int DK>
__device__ __forceinline__ int kchunk_off(int r, int chunk) {
  return r * DK + ((chunk ^ kswz<DK>(r)) << 3);
}

template <typename T, int DK, int DV, bool WITH_V, int NT = 256>
struct KVTile {
  static constexpr bool kVSwz = sizeof(T) == 2;
  static constexpr size_t kElems = (size_t)kTileKeys * DK;
  static constexpr size_t elems = kElems + (WITH_V ? (size_t)DV * (kVSwz ? kTileKeys : kTileVS) : 0);
  // element offset of chunk c (8 keys) of V^T row r
  static __device__ __forceinline__ int voff(int r, int c) {
    if constexpr (kVSwz) return r * kTileKeys + ((c ^ ((r >> 1) & 7)) << 3);
    else return r * kTileVS + c * 8;
  }
  static constexpr int KCH = kTileKeys * DK / 8 / NT;
  static constexpr int VCH = WITH_V ? DV * kTileKeys / 8 / NT : 0;
  static_assert(KCH * NT == kTileKeys * DK / 8, "K tile must split evenly over the workgroup");
  static_assert(!WITH_V || VCH * NT == DV * kTileKeys / 8, "V tile must split evenly over the workgroup");
  Frag8<T> kr[KCH];
  Frag8<T> vr[VCH > 0 ? VCH : 1];

  // key rows: kbase + key * kstride (key clamped to klim-1); V^T rows: vtbase + row * vld.
  __device__ __forceinline__ void gload(const T* kbase, size_t kstride, int klim, const T* vtbase, size_t vld,
                                        int kt) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = threadIdx.x + NT * c, row = idx / (DK / 8), c8 = idx % (DK / 8);
      const int key = min(kt + row, klim - 1);
      kr[c] = load_frag(kbase + (size_t)key * kstride + c8 * 8);
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = threadIdx.x + NT * c, row = idx / (kTileKeys / 8), c8 = idx % (kTileKeys / 8);
      vr[c] = load_frag(vtbase + (size_t)row * vld + kt + c8 * 8);
    }
  }
  __device__ __forceinline__ void lstore(T* tile) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = threadIdx.x + NT * c, row = idx / (DK / 8), c8 = idx % (DK / 8);
      *reinterpret_cast<Frag8<T>*>(tile + kchunk_off<DK>(row, c8)) = kr[c];
    }
    T* vt = tile + kElems;
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = threadIdx.x + NT * c, row = idx / (kTileKeys / 8), c8 = idx % (kTileKeys / 8);
      *reinterpret_cast<Frag8<T>*>(vt + voff(row, c8)) = vr[c];
    }
  }
  // MFMA A operand from the staged K tile: row r of the tile, features ks*32 + qd*8 ..
  static __device__ __forceinline__ Frag8<T> kfrag(const T* tile, int r, int ks, int qd) {
    return *reinterpret_cast<const Frag8<T>*>(tile + kchunk_off<DK>(r, ks * 4 + qd));
  }
  // MFMA A operand of O^T += V^T P^T: V^T row dv, keys k0 + qd*8 ..
  static __device__ __forceinline__ Frag8<T> vfrag(const T* tile, int dv, int k0, int qd) {
    return *reinterpret_cast<const Frag8<T>*>(tile + kElems + voff(dv, k0 / 8 + qd));
  }
};

}  // namespace nsa
