/*
 * attn_fwd.h -- C ABI of the MI355X (gfx950) fused attention forward.
 *
 * The library computes, in one kernel launch per call,
 *
 *     O   = softmax(scale * Q K^T + mask [+ per-head sink in the denominator]) V
 *     lse = log of each row's softmax denominator (natural log)
 *
 * i.e. the attention forward that returns the output together with the per-row
 * log-sum-exp (pith-train pull request 65, "Issues resolved" item 1: FA4's
 * forward returns (out, lse)). Variants covered:
 *
 *   - GQA/MQA: H query heads share Hkv K/V heads, heads kv-major, so query head
 *     h reads K/V head h / (H/Hkv). The query tensor is used as the folded view
 *     [B, Hkv, g*Tq, D] with g = H/Hkv, a reshape and never a copy (ArcFlash
 *     pull request, "What rung 0 does").
 *   - MLA asymmetric head dims d_qk != d_v, the no-rope/rope concatenation done
 *     by the caller (pith-train pull request 65, "Issues resolved" item 2).
 *   - d = 512 heads with attention sinks: a per-head logit that enters each
 *     row's denominator only (ArcFlash pull request, "What rung 0 does").
 *   - A sparse top-k forward in which each query attends to the rows of one
 *     shared KV pool named by its index list (TensorRT-LLM pull request 22028,
 *     "Description": flash_mla_sparse_fwd, 13312 queries x 64 heads x 2176
 *     rows, d_qk 512).
 *
 * Conventions (all calls):
 *   - Ownership: the caller owns every buffer. The library never allocates,
 *     frees or synchronises device memory; it only launches on `stream`.
 *   - Device pointers: q, k, v, kv, out, lse, sinks and indices are device
 *     addresses (hipMalloc or equivalent) and must be 16-byte aligned. Strides
 *     are in ELEMENTS of the tensor's own type; the last dimension is always
 *     contiguous (stride 1). Row strides must keep every row 16-byte aligned.
 *   - Streams: `stream` is a hipStream_t passed as void*. NULL is valid and
 *     means the legacy default stream, as in HIP itself. Calls are
 *     asynchronous with respect to the host.
 *   - Errors: every call returns an attn_status. Argument errors are detected
 *     on the host before anything is launched and leave all buffers untouched;
 *     attn_last_error() then holds a message naming the offending argument.
 *     There is no fallback path: an unsupported shape returns
 *     ATTN_UNSUPPORTED, never a slower kernel.
 *   - Aliasing: out and lse must not overlap any input.
 *   - Thread safety: calls may be made from several host threads; the error
 *     message is per thread and the dispatch counters are atomic.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Versioning. pith-train pull request 65 ("Issues resolved" item 1) records
 * FA4 b19 widening its forward's return tuple from (out, lse) to (out, lse,
 * p, row_max), which broke every caller that unpacked two values. Here no
 * call returns more than a status: every argument struct starts with
 * struct_size (the caller sets it to sizeof the struct it was compiled
 * with; a library built with another layout refuses the call with
 * ATTN_ABI_MISMATCH instead of reading past it), and ATTN_ABI_VERSION is
 * raised whenever any struct or signature changes.
 */
#define ATTN_ABI_VERSION 13

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_INVALID_ARGUMENT = 1, /* null pointer, bad size/stride/alignment, H % Hkv != 0, scale not finite > 0 */
  ATTN_UNSUPPORTED = 2,      /* valid arguments outside the compiled set (head dims, dtype) */
  ATTN_ABI_MISMATCH = 3,     /* struct_size does not match this library */
  ATTN_HIP_ERROR = 4         /* the HIP runtime refused the launch */
} attn_status;

typedef enum attn_dtype {
  ATTN_BF16 = 0, /* bfloat16 inputs and output */
  ATTN_F32 = 1   /* float32 inputs and output (QK^T in split-bf16, see below) */
} attn_dtype;

/*
 * Dense forward arguments.
 *
 *   q   [B, H,   Tq, d_qk]  element strides q_sb, q_sh, q_st (last dim contiguous)
 *   k   [B, Hkv, Tk, d_qk]  strides k_sb, k_sh, k_st
 *   v   [B, Hkv, Tk, d_v]   strides v_sb, v_sh, v_st
 *   out [B, H,   Tq, d_v]   strides o_sb, o_sh, o_st (written)
 *   lse [B, H,   Tq]        float32, contiguous (written)
 *   sinks [H] float32 or NULL. The sink of head h is a logit in the same
 *        space as scale*q.k (it is not multiplied by scale); it adds
 *        exp(sink[h]) to every row's denominator and is included in lse.
 *   causal: 0 or 1. The mask is bottom-right aligned: key j is visible to
 *        query token t iff j <= t + (Tk - Tq). A row that sees no key
 *        gets out = 0 and lse = -inf (lse = sink[h] when sinks are given).
 *   dtype: ATTN_BF16, or ATTN_F32 where q and k are split into a high and
 *        a low bfloat16 part on load so that QK^T keeps ~16 mantissa bits.
 *   Compiled head dims (d_qk, d_v): (64,64), (128,128), (192,128),
 *        (256,256), (512,512) in bf16; (64,64) and (128,128) in f32.
 *   Sizes: B, H, Hkv >= 1, H % Hkv == 0; Tq, Tk >= 0 (Tq == 0 launches nothing;
 *        Tk == 0 writes out = 0 and lse = -inf, or sink).
 *   window_left, window_right: sliding window around each row's diagonal
 *        position c = t + (Tk - Tq): key j is visible only if
 *        j >= c - window_left and j <= c + window_right; -1 leaves that side
 *        unbounded (the window arguments of the FA4 wrappers in
 *        TransformerEngine pull request 3259, "Summary"). The window only
 *        narrows the mask: with causal = 1, window_right has no effect (a
 *        window clamp that widened causal attention to full attention is a
 *        defect the ArcFlash pull request lists under "What this does NOT
 *        do"). bf16 only; (-1, -1) for float32 inputs.
 *   rope_dim, q_rope, k_rope: MLA's two-part query and key without the
 *        concatenation (pith-train pull request 65, "Issues resolved" item
 *        2, builds [q_nope || q_rope] and [k_nope || k_rope] in the model; here
 *        the kernel reads the two parts in place). rope_dim = 0: q and k
 *        hold all d_qk columns (q_rope, k_rope unused). rope_dim > 0: q and
 *        k hold the first d_qk - rope_dim columns, and q_rope [B, H, Tq,
 *        rope_dim] (strides qr_sb, qr_sh, qr_st) and k_rope [B, Hkv, Tk,
 *        rope_dim] (strides kr_sb, kr_sh, kr_st) the last rope_dim; the
 *        result is that of the concatenated rows. kr_sh (and kr_sb) may be
 *        0: one rope key row shared by every kv head, as MLA's decoupled
 *        rope key is. Compiled: bf16, d_qk = 192 with rope_dim = 64, d_v =
 *        128; ATTN_UNSUPPORTED otherwise.
 *   keep, m_sb, m_sh, m_st, p_drop: attention dropout. keep = NULL: none.
 *        Otherwise keep holds the keep bits of every (b, h, t, key): the
 *        32-bit word at keep + b*m_sb + h*m_sh + t*m_st + w (strides in
 *        words, m_st >= ceil(Tk/32)) has bit i set when key 32 w + i is kept.
 *        out = (P * keep / (1 - p_drop)) V; lse is the softmax's, before the
 *        dropout. The caller draws the mask and passes the same one to
 *        attn_bwd_dense, so the two directions cannot disagree on it (the
 *        TransformerEngine pull request 3259 review flags a backward that
 *        lost the forward's dropout state). bf16 with head dims (64,64),
 *        (128,128), (192,128), (256,256), (512,512). Heads up to 256 wide
 *        run a separate, unfused-grade kernel (dispatch path
 *        "dense_dropout_bf16"); (512,512) applies the mask inside the fused
 *        kernel (path "dense_bf16_d512_dropout"). The split-KV, packed and
 *        extra-return calls return ATTN_UNSUPPORTED for it, and so does
 *        attn_plan_dense where the separate kernel would run.
 */
typedef struct attn_dense_args {
  uint32_t struct_size; /* = sizeof(attn_dense_args) */
  int32_t dtype;        /* attn_dtype of q, k, v, out */
  int32_t B, H, Hkv, Tq, Tk, d_qk, d_v;
  int32_t causal;
  float scale;          /* finite, > 0 */
  const void* q;
  int64_t q_sb, q_sh, q_st;
  const void* k;
  int64_t k_sb, k_sh, k_st;
  const void* v;
  int64_t v_sb, v_sh, v_st;
  void* out;
  int64_t o_sb, o_sh, o_st;
  float* lse;
  const float* sinks;
  int32_t window_left;  /* -1: no left bound */
  int32_t window_right; /* -1: no right bound */
  int32_t rope_dim;     /* 0, or the columns held by q_rope / k_rope */
  const void* q_rope;
  int64_t qr_sb, qr_sh, qr_st;
  const void* k_rope;
  int64_t kr_sb, kr_sh, kr_st;
  const uint32_t* keep; /* NULL: no dropout */
  int64_t m_sb, m_sh, m_st;
  float p_drop;         /* in [0, 1) */
} attn_dense_args;

/*
 * Sparse top-k forward arguments.
 *
 *   q       [Sq, Hq, d_qk] bf16, strides q_ss, q_sh
 *   kv      [N, d_qk] bf16, row stride kv_sn: ONE shared pool. The value rows
 *           are its first d_v columns (V == K when d_v == d_qk), so d_v <= d_qk.
 *   indices [Sq, topk] int32, row stride idx_ss. An index outside [0, N)
 *           (canonically -1) is skipped; duplicates count with multiplicity.
 *   out     [Sq, Hq, d_v] bf16, strides o_ss, o_sh (written)
 *   lse     [Sq, Hq] float32, contiguous (written)
 *   sinks   [Hq] float32 or NULL (same meaning as in the dense call)
 *   No mask beyond the index list. Compiled: d_qk = 512 with d_v = 512, 384,
 *   256 or 128 (V is always the first d_v columns of the gathered rows, so each
 *   pool row is still read once), Hq <= 64; other widths return
 *   ATTN_UNSUPPORTED, d_v > d_qk ATTN_INVALID_ARGUMENT (TensorRT-LLM pull
 *   request 22028, "Description": the sparse forward at d_qk 512).
 */
typedef struct attn_sparse_args {
  uint32_t struct_size; /* = sizeof(attn_sparse_args) */
  int32_t dtype;        /* ATTN_BF16 */
  int32_t Sq, Hq, N, d_qk, d_v, topk;
  float scale;
  const void* q;
  int64_t q_ss, q_sh;
  const void* kv;
  int64_t kv_sn;
  const int32_t* indices;
  int64_t idx_ss;
  void* out;
  int64_t o_ss, o_sh;
  float* lse;
  const float* sinks;
} attn_sparse_args;

/*
 * A launch plan, filled on the host without touching the GPU.
 *   path        kernel path name (one path per shape; also the dispatch key)
 *   block_rows  query rows per workgroup (folded rows for dense, heads for sparse)
 *   block_keys  keys per pipeline step
 *   waves       wavefronts per workgroup
 *   grid        workgroups launched
 *   lds_bytes   LDS per workgroup
 *   fold_g      H / Hkv (1 for sparse)
 *   folded_rows g * Tq rows per (b, kv head) of the folded query view
 *   hbm_score_bytes  score bytes written to HBM: 0, the scores stay on chip
 *   budget_tile_rows folded rows per tile if scores of element size
 *               score_elt_bytes were materialised under ATTN_TILE_BYTES
 *               (default 32 MiB): floor(budget / (Tk * elt)) (ArcFlash pull
 *               request, "What rung 0 does": query-row tiling under a budget)
 *   budget_tiles     tiles of that size over all folded rows of one kv head
 */
typedef struct attn_plan {
  uint32_t struct_size; /* = sizeof(attn_plan), set by the caller */
  char path[64];
  int32_t block_rows, block_keys, waves, grid, lds_bytes, fold_g;
  int64_t folded_rows;
  int64_t hbm_score_bytes;
  int64_t budget_bytes;
  int32_t score_elt_bytes;
  int64_t budget_tile_rows;
  int64_t budget_tiles;
} attn_plan;

/* ABI version of the loaded library (ATTN_ABI_VERSION at build time); a
 * binding compares it with the version it was written for before any call
 * (pith-train pull request 65, "Issues resolved" item 1, see above). */
int attn_abi_version(void);

/* Dense forward. Validates, plans and launches one kernel on `stream`. */
attn_status attn_fwd_dense(const attn_dense_args* a, void* stream);

/* Sparse top-k forward. Validates, plans and launches one kernel on `stream`. */
attn_status attn_fwd_sparse_topk(const attn_sparse_args* a, void* stream);

/* The plan attn_fwd_dense / attn_fwd_sparse_topk would launch; host only. */
attn_status attn_plan_dense(const attn_dense_args* a, attn_plan* p);
attn_status attn_plan_sparse_topk(const attn_sparse_args* a, attn_plan* p);

/*
 * Split-KV dense forward, for shapes with few query rows (decode, short
 * prefills) where one workgroup per row block would leave most of the GPU
 * idle. The keys are cut into n ranges of whole key blocks; one launch
 * computes, for every (row block, range), the attention of those rows over
 * that range alone -- O_i normalised by the range's own denominator and
 * lse_i without the sink -- into `workspace`; a second launch merges them:
 *
 *     lse = log(sum_i exp(lse_i) [+ exp(sink[h])]),  O = sum_i exp(lse_i - lse) O_i
 *
 * the output merge of context-parallel attention (TransformerEngine pull
 * request 3259, "Flowchart": ring communication and output merge), here
 * across the workgroups of one device. The result is the same attention as
 * attn_fwd_dense computes (same arguments, same out and lse), up to the
 * rounding of the fp32 partials.
 *
 *   n_splits         key ranges to use, 1..1024 (fewer when there are fewer
 *                    key blocks); 0 lets the library choose: the most
 *                    ranges whose workgroups all fit on the device at once
 *   workspace        device memory, 16-byte aligned, owned by the caller, of
 *                    at least attn_splitkv_workspace_bytes(a, n_splits)
 *                    bytes; its contents on return are unspecified. Calls
 *                    sharing one workspace must be ordered on one stream.
 *   workspace_bytes  its size
 *
 * When the plan needs one range only (few key blocks, Tk == 0, or a grid that
 * already fills the device) this is exactly attn_fwd_dense and the workspace
 * is not touched (NULL allowed). Split ranges are compiled for bf16 inputs:
 * an f32 call with n_splits > 1 returns ATTN_UNSUPPORTED. A workspace that
 * is NULL, misaligned or too small returns ATTN_INVALID_ARGUMENT before any
 * launch. The merge launch is recorded under the dispatch path
 * "splitkv_merge".
 */
attn_status attn_fwd_dense_splitkv(const attn_dense_args* a, int32_t n_splits, void* workspace,
                                   int64_t workspace_bytes, void* stream);

/* Workspace bytes attn_fwd_dense_splitkv needs for these arguments and
 * n_splits (0 = the library's choice): n * B*H*Tq * (d_v + 1) * 4 for n > 1
 * ranges, 0 when one range suffices, -1 on invalid arguments. Host only. */
int64_t attn_splitkv_workspace_bytes(const attn_dense_args* a, int32_t n_splits);

/*
 * The split-KV forward without any allocation, for callers that cannot call
 * hipMalloc or take a workspace from an allocator: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Arguments,
 * range choice and results are those of attn_fwd_dense_splitkv; the partials
 * go to a scratch array the library holds on each device instead of a caller
 * workspace (the caller still passes every input and output). The array is
 * ATTN_NOALLOC_SCRATCH_BYTES (64 MiB) per device, held until the process
 * ends; a plan whose partials need more (attn_splitkv_workspace_bytes)
 * returns ATTN_INVALID_ARGUMENT before any launch -- ask for fewer ranges.
 * Every call on one device shares that device's array: calls that overlap on
 * one device (several streams or host threads) race and must be ordered by
 * the caller. One range only (or f32 inputs with n_splits <= 1) launches the
 * plain kernel and touches no scratch. The call allocates nothing; its first
 * call on a device looks the array's address up (hipGetSymbolAddress), and
 * a failure there returns ATTN_HIP_ERROR.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (64ll << 20)
attn_status attn_fwd_dense_splitkv_noalloc(const attn_dense_args* a, int32_t n_splits, void* stream);

/* The number of key ranges the library would choose (n_splits = 0) for
 * these arguments on the current device; -1 on invalid arguments. Host only
 * (it reads the device's compute-unit count and the kernel's workgroups per
 * CU once; without a device it assumes 256 CUs and the LDS limit). */
int32_t attn_splitkv_choose(const attn_dense_args* a);

/*
 * Dense backward arguments (bf16). The gradients of the dense forward above
 * with respect to q, k, v and the sinks: the raw attention backward that runs
 * after the forward and the output merge in context-parallel training
 * (TransformerEngine pull request 3259, "Flowchart": raw backward -> Q/K/V
 * gradients; "Summary": forward/backward wrappers with LSE handling).
 *
 *   q, k, v  the forward's inputs, layouts and strides as in attn_dense_args
 *   out      [B, H, Tq, d_v] the forward's output O, strides o_sb, o_sh, o_st
 *   dout     [B, H, Tq, d_v] dL/dO, strides do_sb, do_sh, do_st
 *   lse      [B, H, Tq] float32 contiguous: the forward's lse (natural log,
 *            sink included), used to recompute P = exp(scale q.k - lse)
 *   sinks    [H] float32 or NULL, as in the forward
 *   dq       [B, H, Tq, d_qk]  written, strides dq_sb, dq_sh, dq_st
 *   dk       [B, Hkv, Tk, d_qk] written (summed over the g query heads that
 *            read each kv head), strides dk_sb, dk_sh, dk_st
 *   dv       [B, Hkv, Tk, d_v] written, strides dv_sb, dv_sh, dv_st
 *   dsinks   [H] float32 written, or NULL (not computed); must be NULL when
 *            sinks is NULL
 *   causal, scale, sizes, window_left, window_right: as in the forward (the
 *            same values the forward ran with); lse carries no gradient.
 *
 * Gradients are accumulated in fp32 and rounded once to bf16 (dq, dk, dv).
 * No atomics: results are bitwise reproducible. Compiled head dims (d_qk,
 * d_v): (64,64), (128,128), (192,128), (256,256), (512,512); others return
 * ATTN_UNSUPPORTED. The dropout mask (keep) is taken for all of them.
 */
typedef struct attn_dense_bwd_args {
  uint32_t struct_size; /* = sizeof(attn_dense_bwd_args) */
  int32_t dtype;        /* ATTN_BF16 */
  int32_t B, H, Hkv, Tq, Tk, d_qk, d_v;
  int32_t causal;
  float scale;
  const void* q;
  int64_t q_sb, q_sh, q_st;
  const void* k;
  int64_t k_sb, k_sh, k_st;
  const void* v;
  int64_t v_sb, v_sh, v_st;
  const void* out;
  int64_t o_sb, o_sh, o_st;
  const void* dout;
  int64_t do_sb, do_sh, do_st;
  const float* lse;
  const float* sinks;
  void* dq;
  int64_t dq_sb, dq_sh, dq_st;
  void* dk;
  int64_t dk_sb, dk_sh, dk_st;
  void* dv;
  int64_t dv_sb, dv_sh, dv_st;
  float* dsinks;
  int32_t window_left;  /* -1: no left bound */
  int32_t window_right; /* -1: no right bound */
  const uint32_t* keep; /* the forward's dropout mask (see attn_dense_args), or NULL */
  int64_t m_sb, m_sh, m_st;
  float p_drop;
} attn_dense_bwd_args;

/* Workspace bytes attn_bwd_dense needs: B*H*Tq*4 (the row dots
 * rowsum(dO * O)), rounded up to 256; for the 256- and 512-wide heads, where
 * the shape gives fewer than 512 dK/dV workgroups (B*Hkv*ceil(Tk/32) at 512,
 * B*Hkv*ceil(Tk/64) at 256), the query heads of a kv group are split n ways
 * (n = min(H/Hkv, 16, ceil(768 / that count))) and n*B*Hkv*Tk*(d_qk+d_v)*4
 * bytes of fp32 dK/dV partials follow (none when n = 1). -1 on invalid sizes, dtype or head
 * dims (pointers are not examined). Host only. */
int64_t attn_bwd_dense_workspace_bytes(const attn_dense_bwd_args* a);

/* Dense backward: four launches on `stream` (row dots, sink gradients when
 * dsinks != NULL, dK/dV, dQ; a fifth that adds the dK/dV partials in a fixed
 * order when the heads are split, see above). `workspace` is caller-owned device memory,
 * 16-byte aligned, of at least attn_bwd_dense_workspace_bytes(a) bytes; its
 * contents on return are unspecified and calls sharing it must be ordered on
 * one stream. Argument errors (NULL or misaligned pointers, bad strides, a
 * short workspace, dsinks without sinks) return ATTN_INVALID_ARGUMENT before
 * any launch; dtype or head dims outside the compiled set ATTN_UNSUPPORTED.
 * Launches are recorded under the dispatch path "dense_bwd_bf16_d<d_qk>" (with
 * "_v<d_v>" when d_v differs). */
attn_status attn_bwd_dense(const attn_dense_bwd_args* a, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * The forward's extra returns, as a second pass after attn_fwd_dense: FA4 b19
 * widened its forward's return from (out, lse) to (out, lse, p, row_max)
 * (pith-train pull request 65, "Issues resolved" item 1). Read here as
 *   p[b,h,t,j]    = exp(scale * q.k_j - lse[b,h,t]) for visible keys, 0 for
 *                   masked ones (the sink has no column: with sinks a row sums
 *                   to 1 - exp(sink - lse))
 *   row_max[b,h,t] = the largest visible scaled score (the sink is not a
 *                   score); -inf for a row that sees no key.
 * `a` holds the forward's arguments; a->lse is READ here (the forward's lse);
 * v, out and sinks are not used. Masks (causal, window) as in the forward.
 *   p       fp32 [B, H, Tq, Tk] with element strides p_sb, p_sh, p_st (last
 *           dimension contiguous), or NULL
 *   row_max fp32 [B, H, Tq] contiguous, or NULL
 * bf16, d_qk in {64, 128, 192, 256, 512}, rope_dim 0; otherwise
 * ATTN_UNSUPPORTED. One launch on `stream` (dispatch path
 * "dense_extras_bf16"); p costs B*H*Tq*Tk*4 bytes of writes.
 */
attn_status attn_fwd_dense_extras(const attn_dense_args* a, float* p, int64_t p_sb, int64_t p_sh, int64_t p_st,
                                  float* row_max, void* stream);

/*
 * Sparse top-k decode over an fp8 pool: attn_fwd_sparse_topk's result with the
 * pool stored as OCP FP8 E4M3 codes and one fp32 scale per 128 columns of a
 * row (pool value = decoded code * scale; the sparse fp8 decode that the
 * TensorRT-LLM page lists among FlashMLA's kernels). Only the gathered rows
 * are decoded, inside the kernel; the values are the same decoded rows (V ==
 * K, d_v = d). The query's slots are cut into n_splits ranges of whole
 * 32-slot steps (0: the library's choice) whose normalised partial outputs
 * and lse go to the workspace; one merge launch adds the sink and combines.
 *
 *   q      [Sq, Hq, d] bf16, strides q_ss, q_sh (elements)
 *   codes  [N, d] uint8, row stride c_sn (bytes); scales [N, d/128] fp32,
 *          row stride s_sn (elements); N * c_sn and N * s_sn * 4 below 2^32
 *   indices, out, lse, sinks, scale as in attn_fwd_sparse_topk
 *   workspace: attn_sparse_fp8_workspace_bytes(a, n_splits) bytes, 16-byte
 *          aligned, caller-owned
 * Compiled: d = 512, Hq = 64, topk <= 4096 per range. Dispatch path
 * "sparse_fp8_d512" (+ "splitkv_merge").
 */
typedef struct attn_sparse_fp8_args {
  uint32_t struct_size; /* = sizeof(attn_sparse_fp8_args) */
  int32_t Sq, Hq, N, d, topk;
  float scale;
  const void* q;
  int64_t q_ss, q_sh;
  const uint8_t* codes;
  int64_t c_sn;
  const float* scales;
  int64_t s_sn;
  const int32_t* indices;
  int64_t idx_ss;
  void* out;
  int64_t o_ss, o_sh;
  float* lse;
  const float* sinks;
} attn_sparse_fp8_args;

int64_t attn_sparse_fp8_workspace_bytes(const attn_sparse_fp8_args* a, int32_t n_splits);
attn_status attn_fwd_sparse_fp8(const attn_sparse_fp8_args* a, int32_t n_splits, void* workspace,
                                int64_t workspace_bytes, void* stream);

/*
 * Sparse top-k backward: the gradients of attn_fwd_sparse_topk with respect
 * to q, the shared pool and the sinks, from the forward's inputs, its out and
 * lse, and dout = dL/dO (the training counterpart that the rank-1 backward of
 * the pages names beside the dense one; the TensorRT-LLM page, "Description",
 * fixes the forward's shape). With P = exp(scale * q.kv[idx] - lse) and
 * V the pool rows' first d_v columns, the pool row n receives, summed over
 * every (query, slot) whose index is n (a duplicated index twice):
 *   scale * sum_h dS_h q_h  (key role)  +  sum_h P_h dO_h  (value role),
 * with dS = P (dP - rowsum(dO * O)), dP = dO . v.
 *
 *   q, out, dout [Sq, Hq, d] bf16, element strides (q_ss, q_sh) etc.
 *   kv [N, d] bf16 (row stride kv_sn), indices int32 [Sq, topk] (row
 *        stride idx_ss; entries outside [0, N) are skipped as in the forward)
 *   lse [Sq, Hq] fp32 (the forward's), sinks [Hq] fp32 or NULL
 *   dq [Sq, Hq, d] bf16 (written; strides dq_ss, dq_sh)
 *   dkv [N, d] fp32 (overwritten: zeroed, then every contribution added
 *        with fp32 atomics, so the summation order, and the last bits, vary
 *        from run to run); row stride dkv_sn, a multiple of 4
 *   dsinks [Hq] fp32 or NULL (needs sinks)
 *   Compiled: d_qk = d_v = 512, Hq = 64. Workspace: Sq*Hq*4 bytes
 *   (attn_bwd_sparse_workspace_bytes), caller-owned, 16-byte aligned.
 * Launches on `stream`: a fill of dkv, row dots, sink gradients, the
 * gradient kernel (dispatch path "sparse_bwd_bf16_d512"). Errors as for
 * attn_bwd_dense.
 */
typedef struct attn_sparse_bwd_args {
  uint32_t struct_size; /* = sizeof(attn_sparse_bwd_args) */
  int32_t dtype;        /* ATTN_BF16 */
  int32_t Sq, Hq, N, d_qk, d_v, topk;
  float scale;
  const void* q;
  int64_t q_ss, q_sh;
  const void* kv;
  int64_t kv_sn;
  const int32_t* indices;
  int64_t idx_ss;
  const void* out;
  int64_t o_ss, o_sh;
  const void* dout;
  int64_t do_ss, do_sh;
  const float* lse;
  const float* sinks;
  void* dq;
  int64_t dq_ss, dq_sh;
  float* dkv;
  int64_t dkv_sn;
  float* dsinks;
} attn_sparse_bwd_args;

int64_t attn_bwd_sparse_workspace_bytes(const attn_sparse_bwd_args* a);
attn_status attn_bwd_sparse_topk(const attn_sparse_bwd_args* a, void* workspace, int64_t workspace_bytes,
                                 void* stream);

/*
 * Decode forward over a quantized K/V cache. llama.cpp's quantized-KV cache
 * types q8_0 and q4_0 (the llama.cpp page, "Pins #303": the flash-attention
 * kernel dequantizes q4_0 / q8_0 K/V tiles as it loads them, instead of
 * converting the whole cache to f16 every step) are ggml's block formats:
 * rows of d values in blocks of 32, each block an fp16 scale d followed by
 *   ATTN_KV_Q8_0 (ggml type 8): 32 int8 codes q        value = d * q   (34 bytes)
 *   ATTN_KV_Q4_0 (ggml type 2): 16 bytes, byte i holding code i in its low and
 *                               code i + 16 in its high nibble, value = d * (code - 8)
 *                                                                          (18 bytes)
 * The type numbers are ggml's (the page's dispatch census names
 * flash_attn_ext_f16 instances by (ggml_type)8 and (ggml_type)2).
 *
 *   q     [B, H, Tq, d] bf16, element strides q_sb, q_sh, q_st (16-byte rows);
 *         values must lie in the fp16 range (the products run on f16 MFMA)
 *   k, v  [B, Hkv, Tk, d/32 blocks] in kv_format, strides in BYTES (k_sb, k_sh,
 *         k_st, ...; multiples of 4, token stride >= the row's bytes); base
 *         pointers 4-byte aligned
 *   out   [B, H, Tq, d] bf16 (written), lse [B, H, Tq] fp32 contiguous (written)
 *   sinks [H] fp32 or NULL; causal bottom-right as in attn_dense_args.
 *   Compiled: kv_format Q8_0 or Q4_0 (K and V alike), d = 128, 256 or 512
 *   (the head sizes the llama.cpp page's "Overview" lists); other d return
 *   ATTN_UNSUPPORTED.
 *
 * Keys are cut into ranges as in attn_fwd_dense_splitkv (n_splits, 0 = the
 * library's choice; workspace n * B*H*Tq * (d + 1) * 4 bytes from
 * attn_qkv_workspace_bytes, NULL when one range is used) and merged. Errors as
 * in the other calls, before any launch. Launches are recorded under
 * "dense_qkv_<format>_d<d>" ("dense_qkv_q8_0_d128" ... "dense_qkv_q4_0_d512",
 * and "splitkv_merge"); no conversion kernel exists.
 */
typedef enum attn_kv_format { ATTN_KV_Q4_0 = 2, ATTN_KV_Q8_0 = 8 } attn_kv_format;

typedef struct attn_qkv_args {
  uint32_t struct_size; /* = sizeof(attn_qkv_args) */
  int32_t kv_format;    /* attn_kv_format of k and v */
  int32_t B, H, Hkv, Tq, Tk, d;
  int32_t causal;
  float scale;
  const void* q;
  int64_t q_sb, q_sh, q_st; /* elements */
  const void* k;
  int64_t k_sb, k_sh, k_st; /* bytes */
  const void* v;
  int64_t v_sb, v_sh, v_st; /* bytes */
  void* out;
  int64_t o_sb, o_sh, o_st; /* elements */
  float* lse;
  const float* sinks;
} attn_qkv_args;

attn_status attn_fwd_dense_qkv(const attn_qkv_args* a, int32_t n_splits, void* workspace, int64_t workspace_bytes,
                               void* stream);

/* Workspace bytes of attn_fwd_dense_qkv for n_splits (0: the library's
 * choice); 0 when one range suffices, -1 on invalid arguments. Host only. */
int64_t attn_qkv_workspace_bytes(const attn_qkv_args* a, int32_t n_splits);

/*
 * Packed variable-length forward (bf16). The sequences of a batch are laid
 * end to end: sequence b owns query tokens [cu_seqlens_q[b], cu_seqlens_q[b+1])
 * and key tokens [cu_seqlens_k[b], cu_seqlens_k[b+1]). Each sequence is an
 * independent dense attention (bottom-right causal alignment with its own
 * lengths, the same window and sinks); no token attends across a sequence
 * boundary. The ArcFlash pull request ("What this does NOT do") lists a
 * varlen path whose window clamp silently made causal attention full as a
 * defect; here causal applies per sequence.
 *
 *   q     [total_q, H, d_qk], element strides q_st (token), q_sh (head)
 *   k, v  [total_k, Hkv, d], strides k_st, k_sh / v_st, v_sh
 *   out   [total_q, H, d_v] (written), strides o_st, o_sh
 *   lse   [H, total_q] fp32 contiguous (written)
 *   cu_seqlens_q, cu_seqlens_k: device int32 [B + 1], non-decreasing, first
 *         entry 0; entries are clamped to [0, total] on the device, so a
 *         malformed array gives wrong rows, never an out-of-bounds access
 *   max_seqlen_q: the longest query sequence (it sizes the grid; rows of a
 *         longer sequence past it are not computed)
 *   Compiled head dims as for attn_fwd_dense in bf16 with d_qk <= 256 (the
 *   512-wide kernel is built without packed batches: ATTN_UNSUPPORTED); no
 *   split-KV.
 */
typedef struct attn_varlen_args {
  uint32_t struct_size; /* = sizeof(attn_varlen_args) */
  int32_t dtype;        /* ATTN_BF16 */
  int32_t B, H, Hkv, max_seqlen_q, total_q, total_k, d_qk, d_v;
  int32_t causal;
  float scale;
  const void* q;
  int64_t q_st, q_sh;
  const void* k;
  int64_t k_st, k_sh;
  const void* v;
  int64_t v_st, v_sh;
  void* out;
  int64_t o_st, o_sh;
  float* lse;
  const float* sinks;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t window_left;
  int32_t window_right;
} attn_varlen_args;

attn_status attn_fwd_varlen(const attn_varlen_args* a, void* stream);

/* Static text for a status code. */
const char* attn_status_string(attn_status s);

/* Message of the last failed call on this host thread ("" if none). */
const char* attn_last_error(void);

/* Number of launches of kernel path `path` in this process; 0 for a path that
 * never launched or an unknown name. The engagement record of the ArcFlash
 * pull request (section "D18"): a test asserts both that the path it meant to
 * exercise really ran and that the paths it did not mean did not, so a silent
 * fallback cannot pass as the fast path. Counters are atomic and per process. */
uint64_t attn_dispatch_count(const char* path);

/* Reset every dispatch counter to 0 (the same engagement record, "D18"). */
void attn_reset_dispatch_counts(void);

/* Folded query rows per tile when [rows, Tk] scores of elt_bytes each must fit
 * budget_bytes: floor(budget / (Tk * elt)), at least 1; 0 on bad arguments. */
int64_t attn_budget_tile_rows(int64_t budget_bytes, int64_t Tk, int64_t elt_bytes);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_FWD_H */
