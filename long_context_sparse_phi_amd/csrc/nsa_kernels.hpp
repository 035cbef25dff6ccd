// Internal interface between the C ABI layer (nsa_api.cpp) and the kernel
// translation units.  Plain structs of device pointers and sizes; every
// launch_* returns the hipError_t of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nsa {

enum IoType { IO_BF16 = 0, IO_F32 = 1 };

struct Dims {
  int B, T, Hkv, G, Hq, dk, dv;
  int l, d, ls, n, w;
  int ncmp;       // complete compressed blocks of the whole sequence
  int ncmp_pad;   // ncmp rounded up to a multiple of 64 (+64): row stride of V_cmp^T
  int nsel;       // ceil(T / ls)
  int Tp;         // row stride of V^T: T rounded up to 64, plus 64
  int C;          // gate input width
  int Cg;         // gate MLP hidden width (0: one linear gate layer)
  int hidden;     // phi MLP width
  float scale;    // softmax scale
  int io;         // IoType
};

// ---- gate: gates[b,t,h,c] = sigmoid(sum_i x[b,t,i] w[i,h,c]) ----
hipError_t launch_gate(const Dims& dm, int ntok, const void* x, const void* w, float* gates,
                       hipStream_t s);

// ---- transposes ----
// src [B, n, H, D] -> dst [B, H, D, ldd] with zeros in columns n..ldd-1.
hipError_t launch_transpose_seq(const Dims& dm, int B, int n, int H, int D, int ldd,
                                const void* src, void* dst, hipStream_t s);
// src [R, Cc] -> dst [Cc, R]  (element type = io type)
hipError_t launch_transpose_2d(const Dims& dm, int R, int Cc, const void* src, void* dst,
                               hipStream_t s);

// ---- compression phi ----
// mean-pool: x [B,T,Hkv,D] -> out [B,ncmp,Hkv,D]; outT (optional) [B,Hkv,D,ncmp_pad]
hipError_t launch_meanpool(const Dims& dm, int D, const void* x, void* out, void* outT,
                           hipStream_t s);
// MLP phi, in four launches; see nsa_phi.hip.
struct PhiMlpArgs {
  int D;                 // feature dim of this tensor (dk or dv)
  const void* x;         // [B,T,Hkv,D]
  const void* pe;        // [l, D]
  const void* w1;        // [l*D, hidden]
  const void* b1;        // [hidden]
  const void* w2;        // [hidden, D]
  const void* b2;        // [D]
  void* arows;           // ws: [B*Hkv*nsub + l/d, d*D] sub-block rows (io type)
  void* w2t;             // ws: [D, hidden]     (io type)
  float* pe_part;        // ws: position-embedding rows' partial sums (phi_pe_part_floats)
  float* y;              // ws: [B*Hkv*nsub, (l/d)*hidden] sub-block products
  void* h;               // ws: hidden activations [B*Hkv*ncmp, hidden]: bf16 hi,lo pair or fp32
  void* out;             // [B,ncmp,Hkv,D]
  void* outT;            // optional [B,Hkv,D,ncmp_pad]
};
hipError_t launch_phi_mlp(const Dims& dm, const PhiMlpArgs& a, hipStream_t s);
// First phi GEMM alone (sub-block products y, see nsa_phi.hip); arows:
// workspace of (B*Hkv*nsub + l/d) * d*D io elements.
hipError_t launch_phi_gemm1(const Dims& dm, int D, int nsub, const void* x, const void* pe, const void* w1,
                            void* arows, float* y, float* pe_part, hipStream_t s);
// floats of pe_part that launch_phi_gemm1 needs
size_t phi_pe_part_floats(const Dims& dm);
size_t phi_mlp_ws_bytes(const Dims& dm, int D);

// ---- compressed attention ----
struct CmpArgs {
  const void* q;    // [B,T,Hq,dk]
  const void* kc;   // [B,ncmp,Hkv,dk]
  const void* vct;  // [B,Hkv,dv,ncmp_pad]
  float* lse;       // [B,T,Hq]  natural-log lse of the compressed branch
  void* o;          // [B,T,Hq,dv]
  float* p_slc;     // optional [B,T,Hkv,nsel]
  int* idx;         // [B,T,Hkv,n]
  int o_f32;        // o is fp32 (saved for the backward) instead of the I/O type
};
hipError_t launch_cmp_lse(const Dims& dm, const CmpArgs& a, hipStream_t s);
hipError_t launch_cmp_out_topn(const Dims& dm, const CmpArgs& a, hipStream_t s);

// ---- selected attention ----
// K and V in MFMA-fragment order: for every (b, g) and 32-key tile, the
// 2*dk/32 key fragments and dv/16 value fragments a wave loads, each as 64
// lanes x 8 contiguous elements (keys past T are zero).
size_t kv_frag_elems(const Dims& dm);
hipError_t launch_kv_frag(const Dims& dm, const void* k, const void* v, void* kvf, hipStream_t s);
// General form: pack src [B, N, Hkv, D] into tiles of tile_ins instructions,
// as key-row (trans = false, 2*D/32 instructions) or transposed (D/16)
// fragments starting at instruction ins0.
size_t frag_tiles_elems(const Dims& dm, int N, int tile_ins);
hipError_t launch_frag_pack(const Dims& dm, int D, int N, const void* src, void* dst, int tile_ins, int ins0,
                            bool trans, hipStream_t s);

struct SlcArgs {
  const void* q;    // [B,T,Hq,dk]
  const void* kvf;  // fragment-ordered K|V tiles (launch_kv_frag)
  const int* idx;   // [B,T,Hkv,n]
  void* o;          // [B,T,Hq,dv]
  float* lse;       // [B,T,Hq]
  int o_f32;        // o is fp32 instead of the I/O type
};
hipError_t launch_slc(const Dims& dm, const SlcArgs& a, hipStream_t s);
// Gather calibration: k_slc's walk over the same tiles without its arithmetic
// (one word per wave into sink, slc_gather_sink_bytes).
size_t slc_gather_sink_bytes(const Dims& dm);
hipError_t launch_slc_gather(const Dims& dm, const SlcArgs& a, void* sink, hipStream_t s);

// ---- sliding window + gated combine ----
struct WinArgs {
  const void* q;       // [B,T,Hq,dk]
  const void* k;       // [B,T,Hkv,dk]
  const void* vt;      // [B,Hkv,dv,Tp]
  const void* o_cmp;   // [B,T,Hq,dv]
  const void* o_slc;   // [B,T,Hq,dv]
  const float* gates;  // [B,T,Hq,3]
  void* o_win;         // optional [B,T,Hq,dv]
  float* lse;          // optional [B,T,Hq]
  void* o;             // [B,T,Hq,dv]
  int o_f32;           // o_cmp / o_slc / o_win are fp32 instead of the I/O type
  int dense;           // o = window output alone (dense causal attention when w >= T)
};
hipError_t launch_win_combine(const Dims& dm, const WinArgs& a, hipStream_t s);

// Gate MLP (dm.Cg > 0): hid = gelu(x w1 + b1) [ntok, Cg] (pre: before the
// GELU, optional), gates = sigmoid(hid w_gate + b2).  dm.Cg == 0: gates =
// sigmoid(x w_gate).
struct GateMlp {
  const void *w1, *b1, *b2;
};
// Hand-written MFMA GEMM (nsa_gemm.hip): C[m, n] (+)= sum_k A(m, k) B(k, n),
// A(m, k) = A[m*sam + k*sak], B(k, n) = B[k*sbk + n*sbn]; each operand
// k-contiguous or contiguous along its other index, bf16 or fp32 (fp32
// operands enter as bf16 hi + lo parts); C fp32 (optionally accumulated) or
// bf16.  batch independent products, operand and result b offset by b*bsa,
// b*bsb, b*bsc elements.  nsplit > 1 splits k, with batch * nsplit * M * N
// floats of part.
//
// Segments (nseg = 2 or 3, batch 1) make one launch of several products that
// share an operand, the projection layer's q|k|v:
// - along n (seg_k = 0): columns [off, next off) of the product take their B
//   and C from the segment (B(k, n') = B[k*sbk + n'*sbn], C[m*ldc + n'] with
//   n' the column inside the segment); A is the shared operand;
// - along k (seg_k = 1): k in [off, next off) takes A and B from the segment
//   (k' inside the segment); every segment but the last spans a multiple of
//   64, so no k step crosses two; C is shared.
// Every segment's operands have the layout (which index is contiguous) of the
// top-level fields, whose pointers are then unused.  seg[0].off is 0.  With a
// split of k, part holds nsplit * M * N floats, N the total width.
struct MmSeg {
  const void* A; long long sam, sak;
  const void* B; long long sbk, sbn;
  void* C; long long ldc;
  int off;
};
struct MmArgs {
  int M, N, K;
  const void* A; long long sam, sak;
  const void* B; long long sbk, sbn;
  void* C; long long ldc;
  int accumulate;
  int c_bf16;
  int batch = 1;
  long long bsa = 0, bsb = 0, bsc = 0;
  int nseg = 0;
  int seg_k = 0;
  MmSeg seg[3] = {};
};
bool mm_supported(const MmArgs& g, bool a_f32, bool b_f32);
// Exact fp32 GEMM (v_mfma_f32_16x16x4_f32, operands converted to fp32) for
// fp32 I/O and small reductions: C[m*ldc + n] (+)= sum_k A(m, k) B(k, n),
// split over k (at most kGemmMaxSplit ways, nsplit * M * N floats of part)
// when part is given.
struct Gemm {
  int M, N, K;
  const void* A; long long sam, sak;
  const void* B; long long sbk, sbn;
  float* C; long long ldc;
  int accumulate;
};
constexpr int kGemmMaxSplit = 64;
hipError_t gemm_exact(const Gemm& g, bool a_f32, bool b_f32, float* part, hipStream_t s);
int mm_split(const MmArgs& g, int max_split);
hipError_t mm(const MmArgs& g, bool a_f32, bool b_f32, int nsplit, float* part, hipStream_t s);


// dst[i] = float(src[i]) for a bf16 array of n elements.
hipError_t launch_to_f32(const void* src, size_t n, float* dst, hipStream_t s);
hipError_t launch_gate_mlp(const Dims& dm, int ntok, const void* x, const void* w_gate, const GateMlp& g,
                           float* hid, float* pre, float* gates, hipStream_t s);

// Decode-time cache maintenance (nsa_append.hip).  dm.T is the raw cache
// capacity; lens[b] the tokens sequence b held before the call.
struct AppendPhi {
  const void *pe, *w1, *b1, *w2, *b2;
};
struct AppendArgs {
  const int* lens;         // [B]
  const void *kn, *vn;     // [B,Hkv,dk], [B,Hkv,dv]
  void *kc, *vc;           // [B,T,Hkv,dk], [B,T,Hkv,dv]
  // optional per-branch pairs (selected, window): token and raw caches
  // shaped as kn/vn and kc/vc, or all NULL
  const void *kn_slc, *vn_slc, *kn_win, *vn_win;
  void *kc_slc, *vc_slc, *kc_win, *vc_win;
  void *kcmp, *vcmp;       // [B,cap,Hkv,dk], [B,cap,Hkv,dv]
  int cap;
  AppendPhi phi_k, phi_v;
  float* h;                // workspace: first-layer slices [nslice, B*Hkv, hidden]
};
hipError_t launch_append(const Dims& dm, const AppendArgs& a, hipStream_t s);
size_t append_ws_bytes(const Dims& dm);

bool shapes_supported(int dk, int dv);

}  // namespace nsa
