// Launch parameters shared by the host planner (api.cpp) and the gfx950
// kernels (attn_kernels.hip). Plain data only.
#pragma once
#include <stdint.h>

namespace attn {

struct KernelParams {
  const void* q;
  const void* k;        // dense: K; sparse: the shared KV pool
  const void* v;        // dense: V; sparse: same pool (value = first d_v columns)
  void* out;
  float* lse;
  const float* sinks;   // [H] or nullptr
  const int32_t* idx;   // sparse only: [Sq, topk]

  // element strides. dense: (b, h, t); sparse: q (s, h, -), kv row stride in k_st
  int64_t q_sb, q_sh, q_st;
  int64_t k_sb, k_sh, k_st;
  int64_t v_sb, v_sh, v_st;
  int64_t o_sb, o_sh, o_st;
  int64_t idx_ss;
  // two-part q / k rows (kernels compiled with a rope width): the last
  // columns of each row come from q2 / k2 with these strides
  const void* q2;
  const void* k2;
  int64_t q2_sb, q2_sh, q2_st;
  int64_t k2_sb, k2_sh, k2_st;
  // attention dropout inside the fused kernel (512-wide heads): bit k % 32 of
  // keep[b * m_sb + h * m_sh + t * m_st + k / 32] keeps key k of row (b, h, t)
  // in the product with V; the kept probabilities are scaled by inv_keep
  const uint32_t* keep;
  int64_t m_sb, m_sh, m_st;
  float inv_keep;

  int32_t B, H, Hkv, Tq, Tk, g;  // sparse: B = Sq, H = Hq, Hkv = 1, Tk = topk
  int32_t npool;                 // sparse: rows in the pool
  int32_t causal;
  int32_t win_left, win_right;   // sliding window around the diagonal (-1: unbounded side); dense bf16
  float scale;                   // softmax scale
  float c;                       // scale * log2(e)

  // workgroup -> tile decode (dense)
  int32_t aligned;        // 1: tiles never straddle heads (tiles_per_head per head)
  int32_t fold_tm;        // 1 (bf16 kernels, g > 1): token-major fold, row f = t * g + head

  // packed variable-length batch (bf16 kernels): sequence b holds query
  // tokens [cu_q[b], cu_q[b+1]) and key tokens [cu_k[b], cu_k[b+1]) (device
  // arrays, clamped to the totals); Tq / Tk above are the maxima, the batch
  // strides are 0 and lse is [H, total_q]
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t varlen;
  int32_t total_q, total_k;
  int32_t block_rows;     // folded rows per workgroup
  int32_t tiles_per_head; // aligned mode
  int32_t tiles_per_group;// tiles per (b, kv head)
  int32_t n_groups;       // B * Hkv
  int32_t n_tiles;        // grid size
  int32_t xcd_groups;     // 1: workgroup i runs on XCD i % 8; give each XCD whole (b, kv) groups
  int32_t xcd_chunk;      // groups an XCD works on at a time (divides n_groups / 8)

  // split-KV (dense, bf16 paths): blockIdx.y selects keys
  // [y * split_keys, min(Tk, (y + 1) * split_keys)); with n_splits > 1 the
  // kernel writes the partial result of its range (O normalised by its own
  // denominator, fp32, and lse without the sink) to part_o / part_lse
  int32_t n_splits;       // 1: no split
  int32_t split_keys;     // keys per range, a multiple of the kernel's key block
  float* part_o;          // [n_splits][B*H*Tq][d_v]
  float* part_lse;        // [n_splits][B*H*Tq]
};

// Merge of split-KV partials (one launch after the split kernel).
struct MergeParams {
  const float* part_o;
  const float* part_lse;
  const float* sinks;     // [H] or nullptr
  void* out;              // [B, H, Tq, d_v] with the element strides below
  float* lse;             // [B, H, Tq] contiguous
  int64_t o_sb, o_sh, o_st;
  int32_t B, H, Tq, d_v, n_splits;
  int32_t f32;            // 1: out is float32, else bfloat16
};

// Host-side launcher of the merge (defined in attn_kernels.hip).
int launch_merge(const MergeParams& m, void* stream);

// Dense backward (bf16): gradients of q, k, v (and the sinks) from the
// forward's inputs, its output and lse, and the output gradient.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* out;        // forward output O
  const void* dout;       // dL/dO
  const float* lse;       // forward lse [B, H, Tq] contiguous (natural log, sink included)
  const float* sinks;     // [H] or nullptr
  void* dq;
  void* dk;
  void* dv;
  float* dsinks;          // [H] or nullptr
  float* D;               // workspace: rowsum(dO * O), [B, H, Tq]
  // 256- and 512-wide heads with few key blocks: the query heads of a kv group
  // are split n_split ways over workgroups, each writing unscaled fp32 dK and dV
  // partials to part, [n_split, B*Hkv, Tk, 2*d] (dK columns, then dV), summed in
  // split order by a last kernel; n_split = 1 writes dk/dv directly
  float* part;
  int32_t n_split;
  int64_t q_sb, q_sh, q_st, k_sb, k_sh, k_st, v_sb, v_sh, v_st;
  int64_t o_sb, o_sh, o_st, do_sb, do_sh, do_st;
  int64_t dq_sb, dq_sh, dq_st, dk_sb, dk_sh, dk_st, dv_sb, dv_sh, dv_st;
  int32_t B, H, Hkv, Tq, Tk, g;
  int32_t causal;
  int32_t win_left, win_right;  // sliding window as in the forward (-1: unbounded side)
  float scale;
  float c;                // scale * log2(e)
  // dropout (kernels built with it): keep mask bits, word (b, h, t, w) at
  // keep + b*m_sb + h*m_sh + t*m_st + w holds keys 32 w .. 32 w + 31 (bit i =
  // key 32 w + i); kept probabilities are scaled by inv_keep = 1 / (1 - p)
  const uint32_t* keep;
  int64_t m_sb, m_sh, m_st;
  int32_t nwords;         // ceil(Tk / 32)
  float inv_keep;
  void* fwd_out;          // the dropout forward's output [B, H, Tq, d_v] (o strides)
  float* fwd_lse;         // and its lse [B, H, Tq]
  // sparse top-k (launch_bwd_sparse): q, out, dout, dq are [Sq, Hq, 512] with
  // strides (q_sb, q_sh) etc., the pool is k with row stride k_st (values =
  // its first 512 columns), lse / D are [Sq, Hq] (B = Sq, H = Hq, Tq = 1)
  const int32_t* idx;     // [Sq, topk], row stride idx_ss
  int64_t idx_ss;
  int32_t npool, topk;
  float* dkv;             // pool gradient, fp32 [npool, 512], row stride dkv_sn (overwritten)
  int64_t dkv_sn;
};

// Launches the whole backward (row dots, sink gradients, dK/dV, dQ) on
// `stream`; 0 or the hipError_t of a failed launch. Returns -1 when no
// kernel is compiled for (d_qk, d_v).
int launch_bwd(const BwdParams& p, int d_qk, int d_v, void* stream);
// Forward with dropout (p.keep set): one launch writing fwd_out and fwd_lse;
// -1 when no kernel is compiled for (d_qk, d_v) (the backward's set).
int launch_fwd_dropout(const BwdParams& p, int d_qk, int d_v, void* stream);
// (d_qk, d_v) pairs with a compiled backward
bool bwd_supported(int d_qk, int d_v);
// dropout (forward and backward) is compiled for the backward's head dims
bool dropout_supported(int d_qk, int d_v);
// how many ways the 256/512-wide dK/dV kernel splits a kv group's query heads
// (1 for the other widths); the workspace holds the partials when it is > 1
int bwd_head_splits(int B, int Hkv, int g, int Tk, int d_qk, int d_v);
// The forward's extra returns (a second pass from q, k and the forward's
// lse): probabilities of the visible keys and row maxima of the scaled scores.
struct ExtrasParams {
  const void* q;
  const void* k;
  const float* lse;       // [B, H, Tq] contiguous (read)
  float* p;               // [B, H, Tq, Tk] with strides p_sb, p_sh, p_st, or nullptr
  float* row_max;         // [B, H, Tq] contiguous, or nullptr
  int64_t q_sb, q_sh, q_st, k_sb, k_sh, k_st, p_sb, p_sh, p_st;
  int32_t B, H, Hkv, Tq, Tk, g;
  int32_t causal, win_left, win_right;
  float scale, c;
};
int launch_extras(const ExtrasParams& p, int d_qk, void* stream);
bool extras_supported(int d_qk);

// Sparse top-k decode over an fp8 pool (OCP E4M3 codes, one fp32 scale per
// 128 columns of a row; values = the decoded rows, d = 512, 64 heads): the
// query's slots cut into ranges of split_keys (grid y), each writing its
// normalised partial O and lse (no sink) for launch_merge.
struct SpFp8Params {
  const void* q;                 // bf16 [Sq, Hq, 512], strides q_ss, q_sh (elements)
  const unsigned char* codes;    // [N, 512] bytes, row stride c_sn (bytes)
  const float* scales;           // [N, 4], row stride s_sn (elements)
  const int32_t* idx;            // [Sq, topk], row stride idx_ss
  float* part_o;                 // [n_splits][Sq*Hq][512]
  float* part_lse;               // [n_splits][Sq*Hq]
  int64_t q_ss, q_sh, c_sn, s_sn, idx_ss;
  int32_t Sq, Hq, N, topk, split_keys, n_splits;
  float scale, c;
};
int launch_sparse_fp8(const SpFp8Params& p, void* stream);

// Sparse top-k backward (d_qk = d_v = 512, 64 heads): zeroes dkv, then row
// dots, sink gradients and the gradient kernel. 0 or a hipError_t.
int launch_bwd_sparse(const BwdParams& p, void* stream);

// Decode forward over a quantized K/V cache (q8_0 / q4_0 blocks, bf16 q and
// out): the keys of one (b, kv head) and 16 folded query rows per workgroup,
// key ranges on grid y as in split-KV.
struct QkvParams {
  const void* q;
  const unsigned char* k;
  const unsigned char* v;
  void* out;
  float* lse;
  const float* sinks;
  int64_t q_sb, q_sh, q_st;  // elements
  int64_t k_sb, k_sh, k_st;  // bytes
  int64_t v_sb, v_sh, v_st;  // bytes
  int64_t o_sb, o_sh, o_st;  // elements
  int32_t B, H, Hkv, Tq, Tk, g;
  int32_t causal;
  float scale;
  float c;                   // scale * log2(e)
  int32_t n_rt;              // row tiles (16 RT folded rows) per (b, kv head)
  int32_t n_splits, split_keys;
  float* part_o;             // [n_splits][B*H*Tq][d] when n_splits > 1
  float* part_lse;
};

// 16-row tiles a workgroup of the quantized-cache kernel takes (RT) for
// `rows` = g * Tq folded rows of a kv head, format fmt and head dim d
int qkv_row_tiles(int fmt, int d, int rows);
// 0 or the hipError_t of the launch; -1 when (format, d, rt) is not compiled
int launch_qkv(const QkvParams& p, int fmt, int d, int rt, void* stream);
// workgroups of the (format, d, rt) kernel resident on one CU (0: unknown)
int occupancy_qkv(int fmt, int d, int rt);

// Host-side launchers, one per compiled kernel configuration.
// Return 0 on success, else the hipError_t of the launch.
typedef int (*launch_fn)(const KernelParams& p, void* stream);
// workgroups of a kernel that fit on one CU at once (0 when the device cannot be asked)
typedef int (*occupancy_fn)();

struct KernelConfig {
  const char* path;
  int dtype;         // 0 bf16, 1 f32 split
  int d_qk, d_v;
  int sparse;
  int block_rows, block_keys, waves, lds_bytes;
  launch_fn launch;
  occupancy_fn occupancy;
  int rope;          // columns of q / k read from the second pointers (0: none)
  int drop;          // 1: applies the caller's dropout keep mask (KernelParams::keep)
};

// Table of compiled configurations (defined in attn_kernels.hip).
const KernelConfig* kernel_table(int* n);

}  // namespace attn
