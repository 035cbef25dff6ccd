/*
 * nsa.h - C ABI of the MI355X (gfx950) Native Sparse Attention library.
 *
 * The operator (web pages on the NSA paper: youleyou "硬件对齐+原生训练！DeepSeek
 * NSA打造高效稀疏Attention", section 二 整体框架 .. 最终输出计算) replaces the
 * keys/values of each query t by three remapped sets and mixes the three
 * attention outputs with sigmoid gates:
 *     o_t = g_cmp * Attn(q_t, K_cmp, V_cmp) + g_slc * Attn(q_t, K_slc, V_slc)
 *         + g_win * Attn(q_t, K_win, V_win)
 *   cmp: keys/values compressed block-wise by phi over blocks of l tokens
 *        taken every d tokens (令牌压缩), only blocks complete at t;
 *   slc: the tokens (<= t) of the n selection blocks of l' tokens ranked
 *        highest by the compressed branch's probabilities, remapped to
 *        selection blocks and summed over the G query heads of a GQA group
 *        (重要性分数计算, Top-n块选择); block 0 and the two blocks holding
 *        t and the block before are always selected and count inside n;
 *        the lower block index wins a tie;
 *   win: the last w tokens [t-w+1, t] (滑动窗口).
 * Scores use scale / sqrt(d_k) (xookee "NSA论文原理解析", 压缩注意力 §2.4).
 *
 * Conventions shared by every entry point
 * - All tensor pointers are device pointers owned by the caller.  Extra
 *   device memory the kernels need is the caller's workspace of
 *   nsa_workspace_size() bytes.  The library allocates nothing itself; every
 *   kernel, the GEMMs included, is the library's own HIP code (no BLAS
 *   library is called).  The one buffer it holds is the static scratch of
 *   nsa_fwd_decode_noalloc (below), part of the library's code object.
 * - Tensors are dense, row-major, in the order their shapes are written.
 *   Query head h belongs to KV head h / group_size.
 * - io_dtype (NSA_BF16 or NSA_FP32) is the element type of every input and
 *   of o / k_cmp / v_cmp.  o_branch, lse, p_slc, gates and all gradients are
 *   fp32; idx is int32.  Arithmetic accumulates in fp32.
 * - Calls enqueue work on `stream` (a hipStream_t; NULL = default stream)
 *   and return without synchronising.  Results are valid when the stream
 *   reaches that point.
 * - Validation runs before anything is enqueued: on NSA_ERR_INVALID_ARG,
 *   NSA_ERR_UNSUPPORTED or NSA_ERR_WORKSPACE nothing was launched and no
 *   output was touched.  NSA_ERR_HIP reports a failed launch; outputs are
 *   then undefined.  No C++ exception crosses this interface.
 * - Every pointer must be 16-byte aligned.
 * - The device is the caller's current HIP device; it must be gfx950.
 * - Calls on different streams may run concurrently as long as their
 *   buffers do not overlap (nsa_fwd_decode_noalloc excepted, below).  The
 *   only process-wide state is read-only once set: per device, whether it is
 *   a gfx950 and the address of the static scratch buffer.
 */
#ifndef NSA_H_
#define NSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NSA_ABI_VERSION 5

typedef enum nsa_status {
  NSA_OK = 0,
  NSA_ERR_INVALID_ARG = 1,  /* bad shape, hyper-parameter or NULL pointer */
  NSA_ERR_UNSUPPORTED = 2,  /* valid but not built: device, dtype, head dims */
  NSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  NSA_ERR_HIP = 4,          /* a HIP runtime call failed */
  NSA_ERR_INTERNAL = 5,
  /* 6 is not used */
  NSA_ERR_SCRATCH = 7       /* the problem needs more scratch memory than the
                               library's static per-GPU buffer holds
                               (nsa_fwd_decode_noalloc) */
} nsa_status;

typedef enum nsa_dtype { NSA_BF16 = 0, NSA_FP32 = 1 } nsa_dtype;
typedef enum nsa_phi_kind { NSA_PHI_MEANPOOL = 0, NSA_PHI_MLP = 1 } nsa_phi_kind;
typedef enum nsa_op {
  NSA_OP_FWD_PREFILL = 0, NSA_OP_FWD_DECODE = 1, NSA_OP_BWD = 2, NSA_OP_COMPRESS = 3,
  NSA_OP_DENSE = 4, NSA_OP_APPEND = 5, NSA_OP_DENSE_BWD = 6, NSA_OP_LAYER_FWD = 7,
  NSA_OP_LAYER_BWD = 8
} nsa_op;

/* Shapes and hyper-parameters.
 *   batch B; seqlen T (prefill/backward) or cache length S (decode);
 *   n_kv_heads H_kv (H_kv * max(d_k, d_v) < 2^24); group_size G (query heads
 *   per KV head, H_q = H_kv*G, G in {1,2,4,8,16}); d_k, d_v head dims
 *   ((64,64), (128,128), (192,128));
 *   cmp_block l, cmp_stride d (d | l), sel_block l' (d | l', l <= l',
 *   16 | l', l' | 32*d, 31*d + l <= 32*l'); n_select n (3 <= n <= 32);
 *   window w >= 1; gate_dim C (gate input width); phi_hidden (MLP width,
 *   multiple of 64); phi (nsa_phi_kind); io_dtype (nsa_dtype);
 *   scale: 0 selects 1/sqrt(d_k);
 *   gate_hidden: 0 for one linear gate layer, g = sigmoid(x w_gate); otherwise
 *   the width Hg (1 .. 1024) of a two-layer gate MLP (youleyou page,
 *   整体框架: gates from an MLP with a sigmoid),
 *   g = sigmoid(gelu_erf(x w1 + b1) w_gate + b2), weights in nsa_gate_mlp and
 *   w_gate [Hg,Hq,3]. */
typedef struct nsa_params {
  int32_t batch, seqlen, n_kv_heads, group_size, d_k, d_v;
  int32_t cmp_block, cmp_stride, sel_block, n_select, window;
  int32_t gate_dim, phi_hidden;
  int32_t phi;
  int32_t io_dtype;
  float scale;
  int32_t gate_hidden;
} nsa_params;

/* First layer and biases of the gate MLP (io_dtype; used when gate_hidden > 0):
 *   w1 [C, Hg], b1 [Hg], b2 [Hq, 3]. */
typedef struct nsa_gate_mlp {
  const void *w1, *b1, *b2;
} nsa_gate_mlp;

/* Compression MLP phi for keys (D = d_k) or values (D = d_v), io_dtype:
 *   pe [l, D], w1 [l*D, hidden], b1 [hidden], w2 [hidden, D], b2 [D];
 *   block i (tokens i*d .. i*d+l-1): u = concat_j (x[i*d+j] + pe[j]),
 *   phi = gelu_erf(u w1 + b1) w2 + b2.  Ignored for NSA_PHI_MEANPOOL
 *   (phi = mean of the block's l tokens). */
typedef struct nsa_phi_weights {
  const void *pe, *w1, *b1, *w2, *b2;
} nsa_phi_weights;

/* Prefill / training forward.
 * Inputs: q [B,T,Hq,dk], k [B,T,Hkv,dk], v [B,T,Hkv,dv], x [B,T,C],
 *         w_gate [C,Hq,3] (gates g = sigmoid(x w_gate), branch order
 *         cmp, slc, win), phi_k, phi_v.
 * Output: o [B,T,Hq,dv] (required).
 * Optional outputs (NULL = not written; the backward pass needs k_cmp,
 * v_cmp, lse and idx):
 *   k_cmp [B,Ncmp,Hkv,dk], v_cmp [B,Ncmp,Hkv,dv] with Ncmp = (T-l)/d+1
 *     (0 when T < l), rounded to io_dtype;
 *   lse [3,B,T,Hq] fp32 log-sum-exp per branch (-inf for an empty set);
 *   idx [B,T,Hkv,n] int32 selected blocks, ascending, -1 padded;
 *   o_branch [3,B,T,Hq,dv] fp32 per-branch outputs;
 *   p_slc [B,T,Hkv,Nsel] fp32 group importance scores, Nsel = ceil(T/l');
 *   gates [B,T,Hq,3] fp32.
 * Independent keys/values per branch (youleyou page, 滑动窗口: each branch
 * gets its own keys and values so that their gradients do not interfere):
 *   k_slc, v_slc [B,T,Hkv,dk|dv] for the selected branch and k_win, v_win for
 *   the window branch, all four set or all NULL.  When set, k and v feed the
 *   compressed branch (phi) only.  NULL: one k, v for all three branches.
 * Precomputed compressed keys/values (optional, both or neither; the
 * decode step takes its compressed cache the same way):
 *   k_cmp_in [B,Ncmp,Hkv,dk], v_cmp_in [B,Ncmp,Hkv,dv] in io_dtype.  When
 *   set, phi is not run (phi_k, phi_v are not read) and these feed the
 *   compressed branch and the importance scores; k_cmp / v_cmp, if given,
 *   receive a copy of them. */
typedef struct nsa_prefill_args {
  const void *q, *k, *v, *x, *w_gate;
  nsa_phi_weights phi_k, phi_v;
  void *o;
  void *k_cmp, *v_cmp, *lse, *idx, *o_branch, *p_slc, *gates;
  const void *k_slc, *v_slc, *k_win, *v_win;
  nsa_gate_mlp gate_mlp;
  const void *k_cmp_in, *v_cmp_in;
} nsa_prefill_args;

/* One decode step per sequence; the new token's key/value are already stored
 * at cache slot S_b-1 and its query sits at position S_b-1, where S_b is the
 * number of tokens sequence b holds (youleyou page, 效率分析/解码速度: a step
 * reads the compressed blocks, the selected blocks and the window of the
 * cache).
 * Inputs: q [B,Hq,dk], k_cache [B,S,Hkv,dk], v_cache [B,S,Hkv,dv] with
 *   S = p->seqlen (the cache capacity), k_cmp_cache [B,Ncmp_cap,Hkv,dk],
 *   v_cmp_cache [B,Ncmp_cap,Hkv,dv] holding the Ncmp(S_b) = (S_b-l)/d+1
 *   complete compressed blocks of each sequence in their first rows
 *   (cmp_cache_cap = Ncmp_cap >= Ncmp(S)), x [B,C], w_gate.
 *   seq_lens: optional device int32 [B]; NULL means S_b = S for every
 *   sequence.  Values are clamped into [1, S].  Cache rows at or beyond a
 *   sequence's own length (raw rows >= S_b, compressed rows >= Ncmp(S_b))
 *   are never read.
 * Output: o [B,Hq,dv] io_dtype.
 * Optional: idx [B,Hkv,n] int32, p_slc [B,Hkv,Nsel(S)] fp32 (columns at or
 *   beyond Nsel(S_b) = ceil(S_b/l') are written as 0), lse [3,B,Hq] fp32,
 *   o_branch [3,B,Hq,dv] fp32.
 * k_win_cache, v_win_cache: the window branch's own caches [B,S,Hkv,dk|dv]
 *   when each branch has independent keys/values (both set or both NULL);
 *   k_cache, v_cache then serve the selected branch only.
 * A capacity S whose per-(sequence, KV head) score row and per-tile score
 * partials do not fit one compute unit's 160 KB of LDS together returns
 * NSA_ERR_UNSUPPORTED before anything is launched. */
typedef struct nsa_decode_args {
  const void *q, *k_cache, *v_cache, *k_cmp_cache, *v_cmp_cache, *x, *w_gate;
  int32_t cmp_cache_cap;
  void *o;
  void *idx, *p_slc, *lse, *o_branch;
  const int32_t *seq_lens;
  const void *k_win_cache, *v_win_cache;
  nsa_gate_mlp gate_mlp;
} nsa_decode_args;

/* Decode-time cache maintenance: append one token per sequence to the raw
 * caches and keep the compressed caches complete (youleyou page, 令牌压缩:
 * block i covers tokens i*d .. i*d+l-1; it exists once its last token does).
 * For sequence b with L = seq_lens[b] tokens before the call:
 *   k_cache[b, L] = k_new[b], v_cache[b, L] = v_new[b];
 *   if L+1 >= l and (L+1-l) % d == 0, block i = (L+1-l)/d has just become
 *   complete: k_cmp_cache[b, i] = phi_k(k_cache[b, i*d .. i*d+l-1]) and
 *   v_cmp_cache[b, i] = phi_v(...), rounded to io_dtype, exactly as
 *   nsa_compress computes that block.
 * Inputs: k_new [B,Hkv,dk], v_new [B,Hkv,dv] io_dtype; seq_lens device int32
 *   [B] (read only: the caller advances it by one afterwards); phi_k, phi_v
 *   (NSA_PHI_MLP only).
 * In/out: k_cache [B,S,Hkv,dk], v_cache [B,S,Hkv,dv] (S = p->seqlen),
 *   k_cmp_cache [B,cmp_cache_cap,Hkv,dk], v_cmp_cache [B,cmp_cache_cap,Hkv,dv]
 *   with cmp_cache_cap >= Ncmp(S) (NSA_ERR_INVALID_ARG otherwise).
 * Independent keys/values per branch (optional, each quartet all set or all
 *   NULL, else NSA_ERR_INVALID_ARG): k_slc_new [B,Hkv,dk], v_slc_new
 *   [B,Hkv,dv] with k_slc_cache [B,S,Hkv,dk], v_slc_cache [B,S,Hkv,dv] are the
 *   selected branch's token and caches, written as k_slc_cache[b, L] =
 *   k_slc_new[b] (and v); the k_win_* / v_win_* quartet does the same for
 *   the window branch.  k_cache, v_cache then hold the compressed branch's
 *   keys and values, the rows phi reads.  A decode step over such caches takes
 *   k_slc_cache, v_slc_cache as its k_cache, v_cache and k_win_cache,
 *   v_win_cache as its window caches.
 * A sequence whose L is outside [0, S-1] (full cache) is left untouched.
 * No other cache row is written.  Workspace: NSA_OP_APPEND. */
typedef struct nsa_append_args {
  const void *k_new, *v_new;
  const int32_t *seq_lens;
  void *k_cache, *v_cache, *k_cmp_cache, *v_cmp_cache;
  int32_t cmp_cache_cap;
  nsa_phi_weights phi_k, phi_v;
  const void *k_slc_new, *v_slc_new;
  void *k_slc_cache, *v_slc_cache;
  const void *k_win_new, *v_win_new;
  void *k_win_cache, *v_win_cache;
} nsa_append_args;

/* Backward with the selected blocks held fixed (no gradient through the
 * scores or the selection).  Inputs as the prefill forward plus the forward's
 * saved k_cmp, v_cmp, lse, idx and the upstream gradient d_o [B,T,Hq,dv]
 * (io_dtype).  o_branch (optional): the forward's fp32 branch outputs
 * [3,B,T,Hq,dv]; when given, the row terms <dO, O_c> of the softmax backward
 * are read from it (one pass over 3*B*T*Hq*dv floats), otherwise they are
 * recomputed from the probabilities (a second pass over every key).
 * Outputs (fp32, overwritten): dq [B,T,Hq,dk], dk [B,T,Hkv,dk],
 *   dv [B,T,Hkv,dv], dw_gate [C,Hq,3]; for NSA_PHI_MLP also d_phi_k and
 *   d_phi_v laid out like the phi weights (pe, w1, b1, w2, b2) in fp32.
 * Independent keys/values per branch: with k_slc, v_slc, k_win, v_win set
 *   (as in the forward), dk_slc, dv_slc, dk_win, dv_win [B,T,Hkv,dk|dv] fp32
 *   are required and receive those tensors' gradients, and dk, dv hold only
 *   the gradient through the compressed branch (phi).  Without them dk, dv
 *   are the sum over the three branches.
 * Gates: dw_gate is the gradient of w_gate (the gate MLP's output layer when
 *   gate_hidden > 0, then d_gate_mlp receives dw1 [C,Hg], db1 [Hg],
 *   db2 [Hq,3], all required); dx (optional, NULL = not computed) [B,T,C]
 *   fp32 is the gradient with respect to the gate input x. */
typedef struct nsa_phi_grads {
  void *pe, *w1, *b1, *w2, *b2;
} nsa_phi_grads;

typedef struct nsa_gate_grads {
  void *w1, *b1, *b2;
} nsa_gate_grads;

typedef struct nsa_bwd_args {
  const void *q, *k, *v, *x, *w_gate;
  nsa_phi_weights phi_k, phi_v;
  const void *k_cmp, *v_cmp, *lse, *idx, *o_branch, *d_o;
  void *dq, *dk, *dv, *dw_gate;
  nsa_phi_grads d_phi_k, d_phi_v;
  const void *k_slc, *v_slc, *k_win, *v_win;
  void *dk_slc, *dv_slc, *dk_win, *dv_win;
  nsa_gate_mlp gate_mlp;
  nsa_gate_grads d_gate_mlp;
  void *dx;
} nsa_bwd_args;

/* Dense causal attention, the baseline the pages measure NSA against
 * (kernel speed comparison of the youleyou page, 效率分析): for every query
 * head h of KV head h/G,
 *   o[b,t,h] = sum_{j<=t} softmax_j(scale q[b,t,h].k[b,j,h/G]) v[b,j,h/G].
 * Uses batch, seqlen, n_kv_heads, group_size, d_k, d_v, io_dtype and scale of
 * p; the NSA hyper-parameters must still be valid but do not matter.
 * Inputs q [B,T,Hq,dk], k [B,T,Hkv,dk], v [B,T,Hkv,dv]; output o [B,T,Hq,dv]
 * io_dtype; optional lse [B,T,Hq] fp32 natural-log log-sum-exp.  All device
 * pointers, caller-owned, 16-byte aligned.  Workspace: NSA_OP_DENSE. */
typedef struct nsa_dense_args {
  const void *q, *k, *v;
  void *o, *lse;
} nsa_dense_args;

/* Backward of nsa_dense_fwd: with P the causal softmax probabilities and
 * D = <dO, O> per row (the standard attention backward),
 *   dV = P^T dO, dS = P (dO V^T - D), dq = scale dS K, dK = scale dS^T q,
 * summed over the query heads of each KV head.  Inputs q, k, v, the forward's
 * o (io_dtype) and lse ([B,T,Hq] fp32), d_o [B,T,Hq,dv] (io_dtype).  Outputs
 * (fp32, overwritten) dq [B,T,Hq,dk], dk [B,T,Hkv,dk], dv [B,T,Hkv,dv].
 * NSA_ERR_UNSUPPORTED for fp32 with d_k >= 128 (its key tiles do not fit the
 * local memory).  Workspace: NSA_OP_DENSE_BWD. */
typedef struct nsa_dense_bwd_args {
  const void *q, *k, *v, *o, *lse, *d_o;
  void *dq, *dk, *dv;
} nsa_dense_bwd_args;

/* One attention layer around the operator: projections of the layer input to
 * queries, keys and values, NSA with the layer input as the gate input, and
 * the output projection (the module shape of the xookee explainer's
 * 三种注意力如何组合 §2; the youleyou page, 整体框架, derives q, k, v and the
 * gates from the same input):
 *   q = h w_q, k = h w_k, v = h w_v (rounded to io_dtype),
 *   o = NSA(q, k, v; gate input h), y = o w_o (io_dtype).
 * gate_dim C is the layer width.  Inputs (io_dtype, 16-byte aligned):
 *   h [B,T,C], w_q [C, Hq*dk], w_k [C, Hkv*dk], w_v [C, Hkv*dv], w_o [Hq*dv, C],
 *   w_gate, gate_mlp, phi_k, phi_v as for nsa_fwd_prefill.
 * Outputs: y [B,T,C]; q [B,T,Hq,dk], k [B,T,Hkv,dk], v [B,T,Hkv,dv] and
 *   o [B,T,Hq,dv] (io_dtype, required: the backward reads them);
 *   k_cmp, v_cmp, lse, idx, o_branch as nsa_fwd_prefill's (optional; the
 *   backward needs k_cmp, v_cmp, lse and idx).
 * The projections run as the library's bf16 MFMA GEMMs (fp32 accumulation;
 * fp32 I/O: fp32 MFMA) on the stream; with bf16 I/O the width C must be a
 * multiple of 8 (else NSA_ERR_UNSUPPORTED).
 * Workspace: NSA_OP_LAYER_FWD. */
typedef struct nsa_layer_args {
  const void *h, *w_q, *w_k, *w_v, *w_o, *w_gate;
  nsa_gate_mlp gate_mlp;
  nsa_phi_weights phi_k, phi_v;
  void *y, *q, *k, *v, *o;
  void *k_cmp, *v_cmp, *lse, *idx, *o_branch;
} nsa_layer_args;

/* Backward of nsa_layer_fwd with the selected blocks fixed.  Inputs: the
 * forward's inputs, its saved q, k, v, o, k_cmp, v_cmp, lse, idx (o_branch
 * optional, as for nsa_bwd), and dy [B,T,C] io_dtype.  dO = dy w_o^T is
 * rounded to io_dtype (the operator's backward takes dO in io_dtype).
 * Outputs (fp32, overwritten): dh [B,T,C] (through q, k, v and the gate),
 * dw_q, dw_k, dw_v, dw_o (the weights' shapes), dw_gate, d_gate_mlp
 * (gate_hidden > 0), d_phi_k, d_phi_v (NSA_PHI_MLP).
 * Workspace: NSA_OP_LAYER_BWD. */
typedef struct nsa_layer_bwd_args {
  const void *h, *w_q, *w_k, *w_v, *w_o, *w_gate;
  nsa_gate_mlp gate_mlp;
  nsa_phi_weights phi_k, phi_v;
  const void *q, *k, *v, *o, *k_cmp, *v_cmp, *lse, *idx, *o_branch;
  const void *dy;
  void *dh, *dw_q, *dw_k, *dw_v, *dw_o, *dw_gate;
  nsa_gate_grads d_gate_mlp;
  nsa_phi_grads d_phi_k, d_phi_v;
} nsa_layer_bwd_args;

/* Version of this header the library was built from (NSA_ABI_VERSION). */
int nsa_abi_version(void);

/* Static description of a status code; never NULL. */
const char* nsa_status_str(nsa_status s);

/* Workspace bytes entry point `op` needs for `p` (a pure function of p). */
nsa_status nsa_workspace_size(const nsa_params* p, nsa_op op, size_t* bytes);

/* Compress a key or value sequence with phi, as the forward does internally:
 *   x [B,T,Hkv,D] -> out [B,Ncmp,Hkv,D] (io_dtype, Ncmp = (T-l)/d+1).
 * D must equal p->d_k (is_value = 0) or p->d_v (is_value = 1).  Used to
 * build or extend the compressed decode cache.  Workspace: NSA_OP_COMPRESS. */
nsa_status nsa_compress(const nsa_params* p, int is_value, const void* x,
                        const nsa_phi_weights* phi, void* out, void* ws,
                        size_t ws_bytes, void* stream);

nsa_status nsa_fwd_prefill(const nsa_params* p, const nsa_prefill_args* a, void* ws,
                           size_t ws_bytes, void* stream);
nsa_status nsa_fwd_decode(const nsa_params* p, const nsa_decode_args* a, void* ws,
                          size_t ws_bytes, void* stream);

/* The decode step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid allocation.  Same arguments, kernels and results as
 * nsa_fwd_decode; the scratch memory those kernels need (per-chunk softmax
 * states, block scores, selected/window partials) lives in a buffer the
 * library holds in device memory, NSA_DECODE_STATIC_SCRATCH_BYTES per GPU,
 * from the first call on that GPU until the process ends.  The call itself
 * allocates nothing.  A problem whose decode workspace
 * (nsa_workspace_size(p, NSA_OP_FWD_DECODE, ...)) exceeds that size is
 * rejected with NSA_ERR_SCRATCH before anything is enqueued (the 64K-token
 * decode of 32 sequences x 4 KV heads x 16 query heads, d_k = 192, needs
 * about 32 MB).  Every call on one GPU shares that GPU's buffer: calls that
 * may overlap on one GPU (different streams, or different host threads)
 * race and must be ordered by the caller.  Nothing in the buffer needs to
 * start at any value: every value a call reads was written earlier in the
 * same call. */
#define NSA_DECODE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
nsa_status nsa_fwd_decode_noalloc(const nsa_params* p, const nsa_decode_args* a, void* stream);
nsa_status nsa_bwd(const nsa_params* p, const nsa_bwd_args* a, void* ws,
                   size_t ws_bytes, void* stream);
nsa_status nsa_dense_fwd(const nsa_params* p, const nsa_dense_args* a, void* ws,
                         size_t ws_bytes, void* stream);
nsa_status nsa_dense_bwd(const nsa_params* p, const nsa_dense_bwd_args* a, void* ws,
                         size_t ws_bytes, void* stream);
nsa_status nsa_decode_append(const nsa_params* p, const nsa_append_args* a, void* ws,
                             size_t ws_bytes, void* stream);
nsa_status nsa_layer_fwd(const nsa_params* p, const nsa_layer_args* a, void* ws,
                         size_t ws_bytes, void* stream);
nsa_status nsa_layer_bwd(const nsa_params* p, const nsa_layer_bwd_args* a, void* ws,
                         size_t ws_bytes, void* stream);

/* Timed variants, for measurement.  Identical work to the entry points
 * above; in addition hipEventRecord(events[i], stream) is issued before stage
 * i and events[n_stages] after the last stage, so that
 * hipEventElapsedTime(events[i], events[i+1]) is the duration of stage i.
 * `events` holds n_events hipEvent_t created by the caller; n_events must be
 * at least the stage count + 1 (NSA_ERR_INVALID_ARG otherwise).
 * Prefill stages (8): 0 gates, 1 compress K, 2 compress V, 3 transposed V
 *   and fragment-ordered K/V copies,
 *   4 compressed log-sum-exp, 5 compressed output + scores + top-n,
 *   6 selected attention, 7 window attention + gated combine.
 *   With n_events >= stage count + 2, after the last stage the prefill also
 *   runs a gather calibration, timed by events[9]: the selected branch's walk
 *   over the same index rows and fragment-ordered K/V tiles without its
 *   arithmetic (what the memory system takes to deliver that access stream).
 *   It writes only internal workspace; the outputs are those of the stages.
 * Decode stages (3): 0 compressed-cache partial softmax states and scores,
 *   1 combine + group scores + top-n + gates, 2 selected/window attention +
 *   merge + gated combine.
 * Backward stages (8): 0 gates, 1 fragment-ordered copies of (k, v, k^T)
 *   and (k_cmp, v_cmp, k_cmp^T),
 *   2 row terms <dO, O_c> + dq, 3 compressed-key dK/dV, 4 window-key dK/dV,
 *   5 selected-block reverse index + dK/dV, 6 phi backward, 7 dW_g. */
int nsa_prefill_stage_count(void);
int nsa_decode_stage_count(void);
int nsa_bwd_stage_count(void);
nsa_status nsa_fwd_prefill_timed(const nsa_params* p, const nsa_prefill_args* a, void* ws,
                                 size_t ws_bytes, void* stream, void* const* events, int n_events);
nsa_status nsa_fwd_decode_timed(const nsa_params* p, const nsa_decode_args* a, void* ws,
                                size_t ws_bytes, void* stream, void* const* events, int n_events);
nsa_status nsa_bwd_timed(const nsa_params* p, const nsa_bwd_args* a, void* ws, size_t ws_bytes,
                         void* stream, void* const* events, int n_events);

#ifdef __cplusplus
}
#endif
#endif /* NSA_H_ */
