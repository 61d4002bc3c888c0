// Host side of the C ABI declared in include/attn_fwd.h: argument validation,
// the planner (shape -> one kernel path, grid, tile order) and the dispatch
// record. Nothing here allocates or synchronises device memory.
//
// The dispatch record follows the engagement idea of the ArcFlash pull
// request (section "D18 -- engagement asserted, both directions"): every
// launch of a kernel path increments that path's counter, so a test can show
// that the path it meant to exercise really ran, and that a path it did not
// exercise did not.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/attn_fwd.h"
#include "attn_params.h"

namespace {

thread_local std::string g_last_error;

attn_status fail(attn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

constexpr int kMaxPaths = 64;
std::atomic<uint64_t> g_counts[kMaxPaths];
std::atomic<int> g_logged[kMaxPaths];

// the split-KV merge kernel has a counter of its own, after the kernel paths
constexpr int kMergeSlot = kMaxPaths - 1;
constexpr const char* kMergePath = "splitkv_merge";

// the dense backward paths have counters of their own, below the merge's
constexpr const char* kBwdPaths[] = {"dense_bwd_bf16_d64", "dense_bwd_bf16_d128", "dense_bwd_bf16_d192_v128",
                                     "dense_bwd_bf16_d256", "dense_bwd_bf16_d512"};
constexpr int kBwdPathCount = 5;
constexpr int kBwdSlot0 = kMergeSlot - kBwdPathCount;
// and the quantized-cache decode paths below those
constexpr const char* kQkvPaths[] = {"dense_qkv_q8_0_d128", "dense_qkv_q4_0_d128", "dense_qkv_q8_0_d256",
                                     "dense_qkv_q4_0_d256", "dense_qkv_q8_0_d512", "dense_qkv_q4_0_d512"};
constexpr int kQkvPathCount = 6;
constexpr int kQkvSlot0 = kBwdSlot0 - kQkvPathCount;
// and the sparse backward below those
constexpr const char* kSpBwdPath = "sparse_bwd_bf16_d512";
constexpr int kSpBwdSlot = kQkvSlot0 - 1;
constexpr const char* kExtrasPath = "dense_extras_bf16";
constexpr int kExtrasSlot = kSpBwdSlot - 1;
constexpr const char* kDropPath = "dense_dropout_bf16";
constexpr int kDropPathSlot = kExtrasSlot - 1;
constexpr const char* kFp8Path = "sparse_fp8_d512";
constexpr int kFp8Slot = kDropPathSlot - 1;

int path_index(const char* path) {
  if (std::strcmp(path, kMergePath) == 0) return kMergeSlot;
  if (std::strcmp(path, kSpBwdPath) == 0) return kSpBwdSlot;
  if (std::strcmp(path, kExtrasPath) == 0) return kExtrasSlot;
  if (std::strcmp(path, kDropPath) == 0) return kDropPathSlot;
  if (std::strcmp(path, kFp8Path) == 0) return kFp8Slot;
  for (int i = 0; i < kQkvPathCount; ++i)
    if (std::strcmp(path, kQkvPaths[i]) == 0) return kQkvSlot0 + i;
  for (int i = 0; i < kBwdPathCount; ++i)
    if (std::strcmp(path, kBwdPaths[i]) == 0) return kBwdSlot0 + i;
  int n = 0;
  const attn::KernelConfig* t = attn::kernel_table(&n);
  for (int i = 0; i < n && i < kMaxPaths; ++i)
    if (std::strcmp(t[i].path, path) == 0) return i;
  return -1;
}

void note_dispatch(int i, const char* path) {
  g_counts[i].fetch_add(1, std::memory_order_relaxed);
  const char* env = std::getenv("ATTN_LOG_DISPATCH");
  if (env && env[0] == '1' && g_logged[i].exchange(1) == 0)
    std::fprintf(stderr, "attn_fwd: first dispatch on %s\n", path);
}

int64_t tile_budget_bytes() {
  const char* env = std::getenv("ATTN_TILE_BYTES");
  if (env && *env) {
    char* end = nullptr;
    long long v = std::strtoll(env, &end, 10);
    if (end && *end == '\0' && v > 0) return (int64_t)v;
  }
  return (int64_t)32 << 20;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }  // NULL passes

const attn::KernelConfig* find_config(int dtype, int d_qk, int d_v, int sparse, int rope = 0, int drop = 0) {
  int n = 0;
  const attn::KernelConfig* t = attn::kernel_table(&n);
  for (int i = 0; i < n; ++i)
    if (t[i].dtype == dtype && t[i].d_qk == d_qk && t[i].d_v == d_v && t[i].sparse == sparse && t[i].rope == rope &&
        t[i].drop == drop)
      return &t[i];
  return nullptr;
}

// Dropout runs inside the fused kernel for 512-wide heads and as a separate
// kernel for the narrower ones.
bool fused_dropout(const attn_dense_args* a) { return a->keep != nullptr && a->d_qk == 512 && a->d_v == 512; }

struct DensePlan {
  const attn::KernelConfig* cfg;
  attn::KernelParams kp;
  bool drop = false;  // dropout by the separate dropout kernel, not cfg
};

// dropout mask fields shared by the forward and backward argument structs
template <class Args>
static attn_status validate_keep(const Args* a, int Tq, int Tk) {
  if (!a->keep) return ATTN_OK;
  if (a->dtype != ATTN_BF16 || !attn::dropout_supported(a->d_qk, a->d_v))
    return fail(ATTN_UNSUPPORTED,
                "dropout is compiled for bf16 with (d_qk, d_v) in {(64,64), (128,128), (192,128), (256,256), (512,512)}");
  if (!(a->p_drop >= 0.f && a->p_drop < 1.f)) return fail(ATTN_INVALID_ARGUMENT, "p_drop must be in [0, 1)");
  if ((uintptr_t)a->keep & 3u) return fail(ATTN_INVALID_ARGUMENT, "keep must be 4-byte aligned");
  const int64_t nw = ((int64_t)Tk + 31) / 32;
  if (a->m_sb < 0 || a->m_sh < 0 || a->m_st < 0 || (Tq > 1 && a->m_st < nw) || a->m_st >= (1 << 24))
    return fail(ATTN_INVALID_ARGUMENT, "keep strides must be >= 0, m_st >= ceil(Tk/32) and below 2^24 words");
  return ATTN_OK;
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X, each
// with its own L2. When the (batch, kv head) groups split evenly, every XCD
// takes whole groups so that a group's K/V stays in one L2. An XCD runs 32
// workgroups at once (one per CU); it works through its groups a chunk at a
// time, the chunk holding at least `rounds` rounds of its CUs (so the
// longest-first order inside a chunk can balance them), so that concurrent
// workgroups share their K/V in that XCD's L2. Measured: four rounds for
// folded GQA launches (gqa +1.1% over two); one for one-head groups (mla:
// two heads' K/V at a time per L2 fetch 1.55x the algorithmic bytes, four
// 1.8x and eight 2.7x, all in the same time; one head at a time fetches
// 1.0x but runs 10% longer, the last head's longest tiles starting late);
// two for packed batches, whose tiles past a short sequence are empty (four
// cost 11%).
void plan_xcd(attn::KernelParams& p, int rounds = 4) {
  p.xcd_groups = ((p.aligned || p.fold_tm) && p.n_groups % 8 == 0) ? 1 : 0;
  p.xcd_chunk = 0;
  if (!p.xcd_groups) return;
  const int gpx = p.n_groups / 8;
  const int per_group = p.fold_tm ? p.tiles_per_group : p.g * p.tiles_per_head;
  const int want = (32 * rounds + per_group - 1) / per_group;
  int chunk = gpx;
  for (int c = 1; c <= gpx; ++c)
    if (gpx % c == 0 && c >= want) {
      chunk = c;
      break;
    }
  p.xcd_chunk = chunk;
}

attn_status validate_dense(const attn_dense_args* a, DensePlan* out) {
  if (!a) return fail(ATTN_INVALID_ARGUMENT, "args is NULL");
  if (a->struct_size != sizeof(attn_dense_args))
    return fail(ATTN_ABI_MISMATCH, "attn_dense_args.struct_size = %u, library expects %zu", a->struct_size,
                sizeof(attn_dense_args));
  if (a->dtype != ATTN_BF16 && a->dtype != ATTN_F32) return fail(ATTN_UNSUPPORTED, "dtype %d unsupported", a->dtype);
  if (a->B < 1 || a->H < 1 || a->Hkv < 1) return fail(ATTN_INVALID_ARGUMENT, "B, H, Hkv must be >= 1");
  if (a->Tq < 0 || a->Tk < 0) return fail(ATTN_INVALID_ARGUMENT, "Tq, Tk must be >= 0");
  if (a->H % a->Hkv != 0) return fail(ATTN_INVALID_ARGUMENT, "H (%d) must be a multiple of Hkv (%d)", a->H, a->Hkv);
  if (a->d_qk < 1 || a->d_v < 1) return fail(ATTN_INVALID_ARGUMENT, "head dims must be >= 1");
  if (!(std::isfinite(a->scale) && a->scale > 0.f)) return fail(ATTN_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (a->causal != 0 && a->causal != 1) return fail(ATTN_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (a->window_left < -1 || a->window_right < -1)
    return fail(ATTN_INVALID_ARGUMENT, "window bounds must be >= -1 (-1: unbounded)");
  if (a->dtype != ATTN_BF16 && (a->window_left >= 0 || a->window_right >= 0))
    return fail(ATTN_UNSUPPORTED, "sliding windows are compiled for bf16 inputs only");
  if (a->rope_dim < 0 || a->rope_dim >= a->d_qk)
    return fail(ATTN_INVALID_ARGUMENT, "rope_dim must be 0 or in [1, d_qk)");
  const attn::KernelConfig* cfg =
      find_config(a->dtype, a->d_qk, a->d_v, 0, a->rope_dim, a->dtype == ATTN_BF16 && fused_dropout(a) ? 1 : 0);
  if (!cfg)
    return fail(ATTN_UNSUPPORTED, "no compiled dense kernel for dtype %d with (d_qk, d_v) = (%d, %d), rope_dim %d",
                a->dtype, a->d_qk, a->d_v, a->rope_dim);
  const int rope = a->rope_dim;
  const int d_main = a->d_qk - rope;  // columns held by q and k
  {
    const attn_status ks = validate_keep(a, a->Tq, a->Tk);
    if (ks != ATTN_OK) return ks;
    if (a->keep && rope != 0) return fail(ATTN_UNSUPPORTED, "dropout with two-part rows is not compiled");
  }
  if (rope > 0) {
    if (a->Tq > 0 && !a->q_rope) return fail(ATTN_INVALID_ARGUMENT, "q_rope must be non-NULL when Tq > 0");
    if (a->Tk > 0 && !a->k_rope) return fail(ATTN_INVALID_ARGUMENT, "k_rope must be non-NULL when Tk > 0");
    if (!aligned16(a->q_rope) || !aligned16(a->k_rope))
      return fail(ATTN_INVALID_ARGUMENT, "q_rope, k_rope must be 16-byte aligned");
    const int64_t rs[] = {a->qr_sb, a->qr_sh, a->qr_st, a->kr_sb, a->kr_sh, a->kr_st};
    for (int64_t x : rs)
      if (x < 0 || x % 8 != 0)
        return fail(ATTN_INVALID_ARGUMENT, "rope strides must be >= 0 and multiples of 8 elements");
    if (a->kr_st >= (1 << 24)) return fail(ATTN_INVALID_ARGUMENT, "k_rope token stride must be below 2^24 elements");
    if (a->Tq > 1 && a->qr_st < rope) return fail(ATTN_INVALID_ARGUMENT, "q_rope token stride smaller than rope_dim");
    if (a->Tk > 1 && a->kr_st < rope) return fail(ATTN_INVALID_ARGUMENT, "k_rope token stride smaller than rope_dim");
  }
  // empty operands (Tq == 0 or Tk == 0) may come with NULL pointers; they are never read
  if (a->Tq > 0 && (!a->q || !a->out || !a->lse))
    return fail(ATTN_INVALID_ARGUMENT, "q, out, lse must be non-NULL when Tq > 0");
  if (a->Tk > 0 && (!a->k || !a->v)) return fail(ATTN_INVALID_ARGUMENT, "k, v must be non-NULL when Tk > 0");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->out) || !aligned16(a->lse) ||
      !aligned16(a->sinks))
    return fail(ATTN_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  const int64_t vec = (a->dtype == ATTN_BF16) ? 8 : 4;  // elements per 16 bytes
  const int64_t strides[] = {a->q_sb, a->q_sh, a->q_st, a->k_sb, a->k_sh, a->k_st,
                             a->v_sb, a->v_sh, a->v_st, a->o_sb, a->o_sh, a->o_st};
  for (int64_t s : strides)
    if (s < 0 || s % vec != 0)
      return fail(ATTN_INVALID_ARGUMENT, "strides must be >= 0 and keep rows 16-byte aligned (multiple of %lld elements)",
                  (long long)vec);
  if (a->k_st >= (1 << 24) || a->v_st >= (1 << 24))
    return fail(ATTN_INVALID_ARGUMENT, "k/v token strides must be below 2^24 elements");
  if (a->Tq > 1 && a->q_st < d_main) return fail(ATTN_INVALID_ARGUMENT, "q token stride smaller than its row");
  if (a->Tk > 1 && (a->k_st < d_main || a->v_st < a->d_v))
    return fail(ATTN_INVALID_ARGUMENT, "k/v token stride smaller than the head dim");
  if (a->Tq > 1 && a->o_st < a->d_v) return fail(ATTN_INVALID_ARGUMENT, "out token stride smaller than d_v");

  out->cfg = cfg;
  out->drop = a->keep != nullptr && !cfg->drop;
  attn::KernelParams& p = out->kp;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = a->k; p.v = a->v; p.out = a->out; p.lse = a->lse; p.sinks = a->sinks; p.idx = nullptr;
  p.q_sb = a->q_sb; p.q_sh = a->q_sh; p.q_st = a->q_st;
  p.k_sb = a->k_sb; p.k_sh = a->k_sh; p.k_st = a->k_st;
  p.v_sb = a->v_sb; p.v_sh = a->v_sh; p.v_st = a->v_st;
  p.o_sb = a->o_sb; p.o_sh = a->o_sh; p.o_st = a->o_st;
  if (rope > 0) {
    p.q2 = a->q_rope; p.q2_sb = a->qr_sb; p.q2_sh = a->qr_sh; p.q2_st = a->qr_st;
    p.k2 = a->k_rope; p.k2_sb = a->kr_sb; p.k2_sh = a->kr_sh; p.k2_st = a->kr_st;
  }
  p.B = a->B; p.H = a->H; p.Hkv = a->Hkv; p.Tq = a->Tq; p.Tk = a->Tk; p.g = a->H / a->Hkv;
  p.npool = 0;
  p.causal = a->causal;
  p.win_left = a->window_left;
  p.win_right = a->window_right;
  p.scale = a->scale;
  p.c = a->scale * 1.4426950408889634f;
  if (cfg->drop) {
    p.keep = a->keep;
    p.m_sb = a->m_sb; p.m_sh = a->m_sh; p.m_st = a->m_st;
    p.inv_keep = 1.f / (1.f - a->p_drop);
  }
  const int BM = cfg->block_rows;
  p.block_rows = BM;
  p.n_groups = a->B * a->Hkv;
  // Tiles never straddle heads when a head has at least one full block of
  // rows; otherwise the rows of several heads of one group share a tile
  // (the folded view), which is what makes small Tq (decode) efficient.
  const int64_t folded = (int64_t)p.g * a->Tq;
  // bf16 kernels with several heads per kv head fold token-major (row
  // t * g + head): the rows of a tile then span few tokens, so under a
  // causal mask they share almost the same key range and only one key block
  // per tile needs the per-score mask
  p.fold_tm = (cfg->dtype == 0 && p.g > 1) ? 1 : 0;
  // counted in 64 bits before anything is narrowed; the separate dropout
  // kernel tiles the folded rows by 128, so its grid is checked as well
  const int64_t tpg = (!p.fold_tm && a->Tq >= BM) ? (int64_t)((a->Tq + BM - 1) / BM) * p.g : (folded + BM - 1) / BM;
  const int64_t tiles = (int64_t)p.n_groups * tpg;
  const int64_t drop_tiles = out->drop ? (int64_t)p.n_groups * ((folded + 127) / 128) : 0;
  if (tiles > 0x7fffffff || drop_tiles > 0x7fffffff)
    return fail(ATTN_INVALID_ARGUMENT, "problem too large for one launch");
  if (p.fold_tm) {
    p.aligned = 0;
    p.tiles_per_head = 0;
  } else if (a->Tq >= BM) {
    p.aligned = 1;
    p.tiles_per_head = (a->Tq + BM - 1) / BM;
  } else {
    p.aligned = 0;
    p.tiles_per_head = 0;
  }
  p.tiles_per_group = (int)tpg;
  p.n_tiles = (int)tiles;
  plan_xcd(p, p.fold_tm ? 4 : 1);
  return ATTN_OK;
}

attn_status validate_sparse(const attn_sparse_args* a, DensePlan* out) {
  if (!a) return fail(ATTN_INVALID_ARGUMENT, "args is NULL");
  if (a->struct_size != sizeof(attn_sparse_args))
    return fail(ATTN_ABI_MISMATCH, "attn_sparse_args.struct_size = %u, library expects %zu", a->struct_size,
                sizeof(attn_sparse_args));
  if (a->dtype != ATTN_BF16) return fail(ATTN_UNSUPPORTED, "sparse path supports bf16 only");
  if (a->Sq < 0 || a->Hq < 1 || a->N < 1 || a->topk < 0) return fail(ATTN_INVALID_ARGUMENT, "bad Sq/Hq/N/topk");
  if (a->d_v > a->d_qk) return fail(ATTN_INVALID_ARGUMENT, "d_v must not exceed d_qk (V is a prefix of each pool row)");
  if (!(std::isfinite(a->scale) && a->scale > 0.f)) return fail(ATTN_INVALID_ARGUMENT, "scale must be finite and > 0");
  const attn::KernelConfig* cfg = find_config(ATTN_BF16, a->d_qk, a->d_v, 1);
  if (!cfg) return fail(ATTN_UNSUPPORTED, "no compiled sparse kernel for (d_qk, d_v) = (%d, %d)", a->d_qk, a->d_v);
  if (a->Hq > cfg->block_rows)
    return fail(ATTN_UNSUPPORTED, "sparse kernel handles up to %d heads per query, got %d", cfg->block_rows, a->Hq);
  if (a->Sq > 0 && (!a->q || !a->out || !a->lse))
    return fail(ATTN_INVALID_ARGUMENT, "q, out, lse must be non-NULL when Sq > 0");
  if (a->Sq > 0 && a->topk > 0 && (!a->kv || !a->indices))
    return fail(ATTN_INVALID_ARGUMENT, "kv, indices must be non-NULL when Sq > 0 and topk > 0");
  if (!aligned16(a->q) || !aligned16(a->kv) || !aligned16(a->out) || !aligned16(a->lse) ||
      ((uintptr_t)a->indices & 3u) || !aligned16(a->sinks))
    return fail(ATTN_INVALID_ARGUMENT, "device pointers must be 16-byte aligned (indices 4-byte)");
  const int64_t strides[] = {a->q_ss, a->q_sh, a->kv_sn, a->o_ss, a->o_sh};
  for (int64_t s : strides)
    if (s < 0 || s % 8 != 0)
      return fail(ATTN_INVALID_ARGUMENT, "strides must be >= 0 and multiples of 8 elements");
  if (a->kv_sn < a->d_qk) return fail(ATTN_INVALID_ARGUMENT, "kv row stride smaller than d_qk");
  if (a->idx_ss < a->topk) return fail(ATTN_INVALID_ARGUMENT, "index row stride smaller than topk");

  out->cfg = cfg;
  attn::KernelParams& p = out->kp;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = a->kv; p.v = a->kv; p.out = a->out; p.lse = a->lse; p.sinks = a->sinks; p.idx = a->indices;
  p.q_sb = a->q_ss; p.q_sh = a->q_sh;
  p.k_st = a->kv_sn; p.v_st = a->kv_sn;
  p.o_sb = a->o_ss; p.o_sh = a->o_sh;
  p.idx_ss = a->idx_ss;
  p.B = a->Sq; p.H = a->Hq; p.Hkv = 1; p.Tq = 1; p.Tk = a->topk; p.g = 1;
  p.npool = a->N;
  p.win_left = p.win_right = -1;
  p.causal = 0;
  p.scale = a->scale;
  p.c = a->scale * 1.4426950408889634f;
  p.block_rows = cfg->block_rows;
  p.n_groups = a->Sq;
  p.n_tiles = a->Sq;
  return ATTN_OK;
}

void fill_plan(const DensePlan& dp, int fold_g, int64_t folded_rows, int64_t Tk, int score_elt, attn_plan* p) {
  std::memset(reinterpret_cast<char*>(p) + sizeof(p->struct_size), 0, sizeof(*p) - sizeof(p->struct_size));
  std::snprintf(p->path, sizeof(p->path), "%s", dp.cfg->path);
  p->block_rows = dp.cfg->block_rows;
  p->block_keys = dp.cfg->block_keys;
  p->waves = dp.cfg->waves;
  p->grid = dp.kp.n_tiles;
  p->lds_bytes = dp.cfg->lds_bytes;
  p->fold_g = fold_g;
  p->folded_rows = folded_rows;
  p->hbm_score_bytes = 0;  // scores and probabilities never leave the CU
  p->budget_bytes = tile_budget_bytes();
  p->score_elt_bytes = score_elt;
  p->budget_tile_rows = attn_budget_tile_rows(p->budget_bytes, Tk > 0 ? Tk : 1, score_elt);
  p->budget_tiles = p->budget_tile_rows > 0 ? (folded_rows + p->budget_tile_rows - 1) / p->budget_tile_rows : 0;
}

// ---------------------------------------------------------------- split-KV
int device_cus() {
  static std::atomic<int> cached{0};
  int v = cached.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();  // no device here (host-only planning): assume an MI355X
    cus = 256;
  }
  cached.store(cus, std::memory_order_relaxed);
  return cus;
}

constexpr int kMaxSplits = 1024;

struct SplitPlan {
  int n;           // ranges actually launched (1: the plain path)
  int keys;        // keys per range
  int64_t rows;    // B * H * Tq
  int64_t bytes;   // workspace bytes needed (0 when n == 1)
};

// Workgroups of `cfg` resident on one CU at once: the runtime's answer when a
// device is present, else what its LDS allows.
int resident_per_cu(const attn::KernelConfig* cfg) {
  static std::atomic<int> cache[kMaxPaths];
  const int i = path_index(cfg->path);
  int v = (i >= 0) ? cache[i].load(std::memory_order_relaxed) : 0;
  if (v > 0) return v;
  v = cfg->occupancy ? cfg->occupancy() : 0;
  if (v <= 0) v = std::max(1, (160 * 1024) / std::max(1, cfg->lds_bytes));
  if (i >= 0) cache[i].store(v, std::memory_order_relaxed);
  return v;
}

// Ranges of whole key blocks, never more than there are key blocks. The
// library's choice (n_req == 0) is the most ranges whose workgroups all run
// in one round on the device: a second, partial round costs more than the
// longer key loop of fewer, larger ranges, and every range adds partials to
// write and merge.
SplitPlan plan_split(const DensePlan& dp, const attn_dense_args* a, int n_req) {
  SplitPlan sp{1, a->Tk, (int64_t)a->B * a->H * a->Tq, 0};
  const int BN = dp.cfg->block_keys;
  const int nblocks = (a->Tk + BN - 1) / BN;
  if (nblocks <= 1 || a->Tq == 0) return sp;
  int want = n_req;
  if (want == 0) {
    const int64_t slots = (int64_t)device_cus() * resident_per_cu(dp.cfg);
    const int64_t tiles = dp.kp.n_tiles > 0 ? dp.kp.n_tiles : 1;
    want = (int)std::min<int64_t>(kMaxSplits, slots / tiles);
  }
  want = std::min(want, nblocks);
  if (want <= 1) return sp;
  const int per = (nblocks + want - 1) / want;  // key blocks per range
  sp.keys = per * BN;
  sp.n = (a->Tk + sp.keys - 1) / sp.keys;
  if (sp.n <= 1) {
    sp.n = 1;
    sp.keys = a->Tk;
    return sp;
  }
  sp.bytes = (int64_t)sp.n * sp.rows * ((int64_t)a->d_v + 1) * 4;
  return sp;
}

attn_status do_launch(const DensePlan& dp, void* stream) {
  if (dp.kp.n_tiles <= 0) return ATTN_OK;  // nothing to compute (Tq == 0 or Sq == 0)
  const int err = dp.cfg->launch(dp.kp, stream);
  if (err != 0)
    return fail(ATTN_HIP_ERROR, "launch of %s failed: %s", dp.cfg->path, hipGetErrorString((hipError_t)err));
  note_dispatch(path_index(dp.cfg->path), dp.cfg->path);
  return ATTN_OK;
}


// ---------------------------------------------------------------- scratch for callers that cannot allocate
// The partials of attn_fwd_dense_splitkv_noalloc live in this array. Each
// device the library runs on holds its own copy from module load until the
// process ends. Host code never uses the array's name as an address (on the
// host it is only a stand-in symbol): the device address is looked up once
// per device with hipGetSymbolAddress, with that device current, and kept
// below. Every call on a device shares that device's copy, so calls that
// overlap on one device (two streams, two threads) race on it. The kernels
// write every partial they read, so nothing is cleared between calls.
__device__ __attribute__((aligned(256))) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

attn_status scratch_of_current_device(void** out) {
  int dev = -1;
  const hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return fail(ATTN_HIP_ERROR, "hipGetDevice failed: %s", hipGetErrorString(de));
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_UNSUPPORTED, "device %d beyond the %d this library tracks", dev, kMaxDevices);
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || ptr == nullptr)
        return fail(ATTN_HIP_ERROR, "hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
                    hipGetErrorString(e));
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return ATTN_OK;
}

// The split-KV forward: validate, plan the key ranges, launch the ranges and
// the merge. The partials go to the caller's `workspace`
// (attn_fwd_dense_splitkv) or, with `scratch`, to the library's scratch array
// of this device (attn_fwd_dense_splitkv_noalloc; `workspace_bytes` is then
// the array's size, checked before its address is looked up).
attn_status splitkv_launch(const attn_dense_args* a, int32_t n_splits, void* workspace, int64_t workspace_bytes,
                           void* stream, bool scratch) {
  g_last_error.clear();
  DensePlan dp;
  attn_status s = validate_dense(a, &dp);
  if (s != ATTN_OK) return s;
  if (a->keep) return fail(ATTN_UNSUPPORTED, "split-KV with dropout is not compiled");
  if (n_splits < 0 || n_splits > kMaxSplits)
    return fail(ATTN_INVALID_ARGUMENT, "n_splits must be in [0, %d], got %d", kMaxSplits, n_splits);
  if (a->Tq == 0) return ATTN_OK;
  if (a->dtype != ATTN_BF16) {
    if (n_splits > 1) return fail(ATTN_UNSUPPORTED, "split-KV is compiled for bf16 inputs only");
    return do_launch(dp, stream);
  }
  const SplitPlan sp = plan_split(dp, a, n_splits);
  if (sp.n == 1) return do_launch(dp, stream);
  if (scratch) {
    if (sp.bytes > workspace_bytes)
      return fail(ATTN_INVALID_ARGUMENT,
                  "split-KV over %d key ranges needs %lld bytes of partials, more than the %lld bytes of the "
                  "library's scratch array (ask for fewer ranges)",
                  sp.n, (long long)sp.bytes, (long long)workspace_bytes);
    s = scratch_of_current_device(&workspace);
    if (s != ATTN_OK) return s;
  }
  if (workspace == nullptr || workspace_bytes < sp.bytes)
    return fail(ATTN_INVALID_ARGUMENT, "split-KV over %d key ranges needs a workspace of %lld bytes, got %lld", sp.n,
                (long long)sp.bytes, (long long)(workspace ? workspace_bytes : 0));
  if (!aligned16(workspace)) return fail(ATTN_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  attn::KernelParams& p = dp.kp;
  p.n_splits = sp.n;
  p.split_keys = sp.keys;
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = p.part_o + (int64_t)sp.n * sp.rows * a->d_v;
  s = do_launch(dp, stream);
  if (s != ATTN_OK) return s;
  attn::MergeParams m;
  m.part_o = p.part_o;
  m.part_lse = p.part_lse;
  m.sinks = a->sinks;
  m.out = a->out;
  m.lse = a->lse;
  m.o_sb = a->o_sb; m.o_sh = a->o_sh; m.o_st = a->o_st;
  m.B = a->B; m.H = a->H; m.Tq = a->Tq; m.d_v = a->d_v; m.n_splits = sp.n;
  m.f32 = 0;
  const int err = attn::launch_merge(m, stream);
  if (err != 0) return fail(ATTN_HIP_ERROR, "launch of the split-KV merge failed: %s", hipGetErrorString((hipError_t)err));
  note_dispatch(kMergeSlot, kMergePath);
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

static attn_status launch_dropout(const attn_dense_args* a, void* stream) {
  attn::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = a->k; p.v = a->v; p.sinks = a->sinks;
  p.fwd_out = a->out; p.fwd_lse = a->lse;
  p.q_sb = a->q_sb; p.q_sh = a->q_sh; p.q_st = a->q_st;
  p.k_sb = a->k_sb; p.k_sh = a->k_sh; p.k_st = a->k_st;
  p.v_sb = a->v_sb; p.v_sh = a->v_sh; p.v_st = a->v_st;
  p.o_sb = a->o_sb; p.o_sh = a->o_sh; p.o_st = a->o_st;
  p.B = a->B; p.H = a->H; p.Hkv = a->Hkv; p.Tq = a->Tq; p.Tk = a->Tk; p.g = a->H / a->Hkv;
  p.causal = a->causal; p.win_left = a->window_left; p.win_right = a->window_right;
  p.scale = a->scale;
  p.c = a->scale * 1.4426950408889634f;
  p.keep = a->keep; p.m_sb = a->m_sb; p.m_sh = a->m_sh; p.m_st = a->m_st;
  p.nwords = (int)(((int64_t)a->Tk + 31) / 32);
  p.inv_keep = 1.f / (1.f - a->p_drop);
  const int err = attn::launch_fwd_dropout(p, a->d_qk, a->d_v, stream);
  if (err != 0) return fail(ATTN_HIP_ERROR, "launch of the dropout forward failed: %s", hipGetErrorString((hipError_t)err));
  note_dispatch(kDropPathSlot, kDropPath);
  return ATTN_OK;
}

attn_status attn_fwd_dense(const attn_dense_args* a, void* stream) {
  g_last_error.clear();
  DensePlan dp;
  attn_status s = validate_dense(a, &dp);
  if (s != ATTN_OK) return s;
  if (a->Tq == 0) return ATTN_OK;
  if (dp.drop) return launch_dropout(a, stream);
  return do_launch(dp, stream);
}

attn_status attn_fwd_sparse_topk(const attn_sparse_args* a, void* stream) {
  g_last_error.clear();
  DensePlan dp;
  attn_status s = validate_sparse(a, &dp);
  if (s != ATTN_OK) return s;
  return do_launch(dp, stream);
}

attn_status attn_plan_dense(const attn_dense_args* a, attn_plan* p) {
  g_last_error.clear();
  if (!p) return fail(ATTN_INVALID_ARGUMENT, "plan is NULL");
  if (p->struct_size != sizeof(attn_plan))
    return fail(ATTN_ABI_MISMATCH, "attn_plan.struct_size = %u, library expects %zu", p->struct_size, sizeof(attn_plan));
  DensePlan dp;
  attn_status s = validate_dense(a, &dp);
  if (s != ATTN_OK) return s;
  if (dp.drop) return fail(ATTN_UNSUPPORTED, "plans describe the fused kernels; dropout at this width runs a separate kernel");
  if (a->Tq == 0) dp.kp.n_tiles = 0;
  fill_plan(dp, a->H / a->Hkv, (int64_t)(a->H / a->Hkv) * a->Tq, a->Tk, a->dtype == ATTN_BF16 ? 2 : 4, p);
  return ATTN_OK;
}

int32_t attn_splitkv_choose(const attn_dense_args* a) {
  g_last_error.clear();
  DensePlan dp;
  if (validate_dense(a, &dp) != ATTN_OK) return -1;
  if (a->keep) {
    fail(ATTN_UNSUPPORTED, "split-KV with dropout is not compiled");
    return -1;
  }
  if (a->dtype != ATTN_BF16) return 1;
  return plan_split(dp, a, 0).n;
}

int64_t attn_splitkv_workspace_bytes(const attn_dense_args* a, int32_t n_splits) {
  g_last_error.clear();
  DensePlan dp;
  if (validate_dense(a, &dp) != ATTN_OK) return -1;
  if (a->keep) {
    fail(ATTN_UNSUPPORTED, "split-KV with dropout is not compiled");
    return -1;
  }
  if (n_splits < 0 || n_splits > kMaxSplits) {
    fail(ATTN_INVALID_ARGUMENT, "n_splits must be in [0, %d], got %d", kMaxSplits, n_splits);
    return -1;
  }
  if (a->dtype != ATTN_BF16) return 0;
  return plan_split(dp, a, n_splits).bytes;
}

attn_status attn_fwd_dense_splitkv(const attn_dense_args* a, int32_t n_splits, void* workspace,
                                   int64_t workspace_bytes, void* stream) {
  return splitkv_launch(a, n_splits, workspace, workspace_bytes, stream, false);
}

attn_status attn_fwd_dense_splitkv_noalloc(const attn_dense_args* a, int32_t n_splits, void* stream) {
  return splitkv_launch(a, n_splits, nullptr, ATTN_NOALLOC_SCRATCH_BYTES, stream, true);
}

attn_status attn_plan_sparse_topk(const attn_sparse_args* a, attn_plan* p) {
  g_last_error.clear();
  if (!p) return fail(ATTN_INVALID_ARGUMENT, "plan is NULL");
  if (p->struct_size != sizeof(attn_plan))
    return fail(ATTN_ABI_MISMATCH, "attn_plan.struct_size = %u, library expects %zu", p->struct_size, sizeof(attn_plan));
  DensePlan dp;
  attn_status s = validate_sparse(a, &dp);
  if (s != ATTN_OK) return s;
  fill_plan(dp, 1, a->Hq, a->topk, 2, p);
  return ATTN_OK;
}

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_INVALID_ARGUMENT: return "invalid argument";
    case ATTN_UNSUPPORTED: return "unsupported";
    case ATTN_ABI_MISMATCH: return "ABI mismatch";
    case ATTN_HIP_ERROR: return "HIP error";
  }
  return "unknown status";
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------- dense backward
namespace {

static int bwd_path(int d_qk, int d_v) {
  if (d_qk == 64 && d_v == 64) return 0;
  if (d_qk == 128 && d_v == 128) return 1;
  if (d_qk == 192 && d_v == 128) return 2;
  if (d_qk == 256 && d_v == 256) return 3;
  if (d_qk == 512 && d_v == 512) return 4;
  return -1;
}

// sizes, dtype and head dims only (what the workspace size depends on)
static attn_status validate_bwd_shape(const attn_dense_bwd_args* a) {
  if (!a) return fail(ATTN_INVALID_ARGUMENT, "args is NULL");
  if (a->struct_size != sizeof(attn_dense_bwd_args))
    return fail(ATTN_ABI_MISMATCH, "attn_dense_bwd_args.struct_size = %u, library expects %zu", a->struct_size,
                sizeof(attn_dense_bwd_args));
  if (a->dtype != ATTN_BF16) return fail(ATTN_UNSUPPORTED, "the backward is compiled for bf16 only (dtype %d)", a->dtype);
  if (a->B < 1 || a->H < 1 || a->Hkv < 1) return fail(ATTN_INVALID_ARGUMENT, "B, H, Hkv must be >= 1");
  if (a->Tq < 0 || a->Tk < 0) return fail(ATTN_INVALID_ARGUMENT, "Tq, Tk must be >= 0");
  if (a->H % a->Hkv != 0) return fail(ATTN_INVALID_ARGUMENT, "H (%d) must be a multiple of Hkv (%d)", a->H, a->Hkv);
  if (a->d_qk < 1 || a->d_v < 1) return fail(ATTN_INVALID_ARGUMENT, "head dims must be >= 1");
  if (!(std::isfinite(a->scale) && a->scale > 0.f)) return fail(ATTN_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (a->causal != 0 && a->causal != 1) return fail(ATTN_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (a->window_left < -1 || a->window_right < -1)
    return fail(ATTN_INVALID_ARGUMENT, "window bounds must be >= -1 (-1: unbounded)");
  if (bwd_path(a->d_qk, a->d_v) < 0)
    return fail(ATTN_UNSUPPORTED, "no compiled dense backward for (d_qk, d_v) = (%d, %d)", a->d_qk, a->d_v);
  // one-dimensional grids: (key blocks or row tiles) x B x Hkv workgroups;
  // counted with the smallest blocks of any path (32 keys, up to 16 head
  // splits; 32 folded rows)
  const int64_t groups = (int64_t)a->B * a->Hkv;
  const int64_t tiles = std::max<int64_t>((a->Tk + 31) / 32 * 16, ((int64_t)(a->H / a->Hkv) * a->Tq + 31) / 32);
  if (groups * tiles > 0x7fffffff) return fail(ATTN_UNSUPPORTED, "problem too large for one launch");
  return ATTN_OK;
}

static attn_status validate_bwd(const attn_dense_bwd_args* a) {
  const attn_status s = validate_bwd_shape(a);
  if (s != ATTN_OK) return s;
  if (a->Tq > 0 && (!a->q || !a->out || !a->dout || !a->lse || !a->dq))
    return fail(ATTN_INVALID_ARGUMENT, "q, out, dout, lse, dq must be non-NULL when Tq > 0");
  if (a->Tk > 0 && (!a->k || !a->v || !a->dk || !a->dv))
    return fail(ATTN_INVALID_ARGUMENT, "k, v, dk, dv must be non-NULL when Tk > 0");
  if (a->dsinks && !a->sinks) return fail(ATTN_INVALID_ARGUMENT, "dsinks given without sinks");
  const void* ptrs[] = {a->q, a->k, a->v, a->out, a->dout, a->lse, a->sinks, a->dq, a->dk, a->dv, a->dsinks};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return fail(ATTN_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  const int64_t strides[] = {a->q_sb,  a->q_sh,  a->q_st,  a->k_sb,  a->k_sh,  a->k_st,  a->v_sb,  a->v_sh,
                             a->v_st,  a->o_sb,  a->o_sh,  a->o_st,  a->do_sb, a->do_sh, a->do_st, a->dq_sb,
                             a->dq_sh, a->dq_st, a->dk_sb, a->dk_sh, a->dk_st, a->dv_sb, a->dv_sh, a->dv_st};
  for (int64_t s : strides)
    if (s < 0 || s % 8 != 0)
      return fail(ATTN_INVALID_ARGUMENT, "strides must be >= 0 and keep rows 16-byte aligned (multiple of 8 elements)");
  if (a->q_st >= (1 << 24) || a->do_st >= (1 << 24) || a->k_st >= (1 << 24) || a->v_st >= (1 << 24))
    return fail(ATTN_INVALID_ARGUMENT, "q, dout, k, v token strides must be below 2^24 elements");
  if (a->Tq > 1 && (a->q_st < a->d_qk || a->dq_st < a->d_qk || a->o_st < a->d_v || a->do_st < a->d_v))
    return fail(ATTN_INVALID_ARGUMENT, "query-side token stride smaller than the head dim");
  if (a->Tk > 1 && (a->k_st < a->d_qk || a->v_st < a->d_v || a->dk_st < a->d_qk || a->dv_st < a->d_v))
    return fail(ATTN_INVALID_ARGUMENT, "key-side token stride smaller than the head dim");
  return validate_keep(a, a->Tq, a->Tk);
}

// the row dots D (fp32 [B, H, Tq]), then, where the dK/dV kernel splits the
// query heads of a kv group, its fp32 partials [n_split, B*Hkv, Tk, d_qk + d_v]
static int64_t bwd_dots_bytes(const attn_dense_bwd_args* a) {
  const int64_t rows = (int64_t)a->B * a->H * a->Tq;
  return (rows * 4 + 255) / 256 * 256;
}

static int bwd_splits(const attn_dense_bwd_args* a) {
  return attn::bwd_head_splits(a->B, a->Hkv, a->H / a->Hkv, a->Tk, a->d_qk, a->d_v);
}

static int64_t bwd_workspace(const attn_dense_bwd_args* a) {
  const int ns = bwd_splits(a);
  const int64_t part = ns > 1 ? (int64_t)ns * a->B * a->Hkv * a->Tk * (a->d_qk + a->d_v) * 4 : 0;
  return bwd_dots_bytes(a) + part;
}

}  // namespace

int64_t attn_bwd_dense_workspace_bytes(const attn_dense_bwd_args* a) {
  g_last_error.clear();
  if (validate_bwd_shape(a) != ATTN_OK) return -1;
  return bwd_workspace(a);
}

attn_status attn_bwd_dense(const attn_dense_bwd_args* a, void* workspace, int64_t workspace_bytes, void* stream) {
  g_last_error.clear();
  attn_status s = validate_bwd(a);
  if (s != ATTN_OK) return s;
  const int64_t need = bwd_workspace(a);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(ATTN_INVALID_ARGUMENT, "the backward needs a workspace of %lld bytes, got %lld", (long long)need,
                (long long)(workspace ? workspace_bytes : 0));
  if (!aligned16(workspace)) return fail(ATTN_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  attn::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = a->k; p.v = a->v; p.out = a->out; p.dout = a->dout; p.lse = a->lse; p.sinks = a->sinks;
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv; p.dsinks = a->dsinks;
  p.D = static_cast<float*>(workspace);
  p.n_split = bwd_splits(a);
  p.part = p.n_split > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_dots_bytes(a)) : nullptr;
  p.q_sb = a->q_sb; p.q_sh = a->q_sh; p.q_st = a->q_st;
  p.k_sb = a->k_sb; p.k_sh = a->k_sh; p.k_st = a->k_st;
  p.v_sb = a->v_sb; p.v_sh = a->v_sh; p.v_st = a->v_st;
  p.o_sb = a->o_sb; p.o_sh = a->o_sh; p.o_st = a->o_st;
  p.do_sb = a->do_sb; p.do_sh = a->do_sh; p.do_st = a->do_st;
  p.dq_sb = a->dq_sb; p.dq_sh = a->dq_sh; p.dq_st = a->dq_st;
  p.dk_sb = a->dk_sb; p.dk_sh = a->dk_sh; p.dk_st = a->dk_st;
  p.dv_sb = a->dv_sb; p.dv_sh = a->dv_sh; p.dv_st = a->dv_st;
  p.B = a->B; p.H = a->H; p.Hkv = a->Hkv; p.Tq = a->Tq; p.Tk = a->Tk; p.g = a->H / a->Hkv;
  p.causal = a->causal;
  p.win_left = a->window_left;
  p.win_right = a->window_right;
  p.scale = a->scale;
  p.c = a->scale * 1.4426950408889634f;
  if (a->keep) {
    p.keep = a->keep; p.m_sb = a->m_sb; p.m_sh = a->m_sh; p.m_st = a->m_st;
    p.nwords = (int)(((int64_t)a->Tk + 31) / 32);
    p.inv_keep = 1.f / (1.f - a->p_drop);
  }
  const int err = attn::launch_bwd(p, a->d_qk, a->d_v, stream);
  if (err != 0)
    return fail(ATTN_HIP_ERROR, "launch of the dense backward failed: %s", hipGetErrorString((hipError_t)err));
  const int bp = bwd_path(a->d_qk, a->d_v);
  note_dispatch(kBwdSlot0 + bp, kBwdPaths[bp]);
  return ATTN_OK;
}

// ---------------------------------------------------------------- the forward's extra returns
attn_status attn_fwd_dense_extras(const attn_dense_args* a, float* p_out, int64_t p_sb, int64_t p_sh, int64_t p_st,
                                  float* row_max, void* stream) {
  g_last_error.clear();
  DensePlan dp;
  attn_status st = validate_dense(a, &dp);
  if (st != ATTN_OK) return st;
  if (a->keep) return fail(ATTN_UNSUPPORTED, "the extra returns take no dropout mask");
  if (a->dtype != ATTN_BF16 || a->rope_dim != 0 || !attn::extras_supported(a->d_qk))
    return fail(ATTN_UNSUPPORTED, "the extra returns are compiled for bf16, d_qk in {64,128,192,256,512}, rope_dim 0");
  if (((uintptr_t)p_out & 3u) || ((uintptr_t)row_max & 3u))
    return fail(ATTN_INVALID_ARGUMENT, "p and row_max must be 4-byte aligned");
  if (p_out && (p_sb < 0 || p_sh < 0 || p_st < 0 || (a->Tq > 1 && p_st < a->Tk)))
    return fail(ATTN_INVALID_ARGUMENT, "p strides must be >= 0 with a token stride of at least Tk");
  if (a->Tq == 0 || (!p_out && !row_max)) return ATTN_OK;
  attn::ExtrasParams e;
  std::memset(&e, 0, sizeof(e));
  e.q = a->q; e.k = a->k; e.lse = a->lse; e.p = p_out; e.row_max = row_max;
  e.q_sb = a->q_sb; e.q_sh = a->q_sh; e.q_st = a->q_st;
  e.k_sb = a->k_sb; e.k_sh = a->k_sh; e.k_st = a->k_st;
  e.p_sb = p_sb; e.p_sh = p_sh; e.p_st = p_st;
  e.B = a->B; e.H = a->H; e.Hkv = a->Hkv; e.Tq = a->Tq; e.Tk = a->Tk; e.g = a->H / a->Hkv;
  e.causal = a->causal; e.win_left = a->window_left; e.win_right = a->window_right;
  e.scale = a->scale;
  e.c = a->scale * 1.4426950408889634f;
  const int err = attn::launch_extras(e, a->d_qk, stream);
  if (err != 0) return fail(ATTN_HIP_ERROR, "launch of the extra returns failed: %s", hipGetErrorString((hipError_t)err));
  note_dispatch(kExtrasSlot, kExtrasPath);
  return ATTN_OK;
}

// ---------------------------------------------------------------- sparse decode over an fp8 pool
namespace {

struct Fp8Plan {
  int n, split_keys;
  int64_t bytes;
};

static attn_status validate_fp8_shape(const attn_sparse_fp8_args* a) {
  if (!a) return fail(ATTN_INVALID_ARGUMENT, "args is NULL");
  if (a->struct_size != sizeof(attn_sparse_fp8_args))
    return fail(ATTN_ABI_MISMATCH, "attn_sparse_fp8_args.struct_size = %u, library expects %zu", a->struct_size,
                sizeof(attn_sparse_fp8_args));
  if (a->Sq < 0 || a->Hq < 1 || a->N < 1 || a->topk < 0) return fail(ATTN_INVALID_ARGUMENT, "bad Sq/Hq/N/topk");
  if (a->d != 512 || a->Hq != 64)
    return fail(ATTN_UNSUPPORTED, "the fp8 sparse decode is compiled for d = 512 and Hq = 64 (got %d, %d)", a->d, a->Hq);
  if (!(std::isfinite(a->scale) && a->scale > 0.f)) return fail(ATTN_INVALID_ARGUMENT, "scale must be finite and > 0");
  return ATTN_OK;
}

// ranges of whole 32-slot steps: enough workgroups for one per CU (a
// workgroup takes 146 KiB of LDS; measured at 128 queries: two ranges 103 us,
// four 116 us, three 130 us), at most 4096 slots (the kernel's index buffer)
// per range
static Fp8Plan plan_fp8(const attn_sparse_fp8_args* a, int n_req) {
  Fp8Plan pl;
  const int steps = std::max(1, (a->topk + 31) / 32);
  int n = n_req;
  if (n <= 0) n = std::max(1, (device_cus() + std::max(a->Sq, 1) - 1) / std::max(a->Sq, 1));
  n = std::max(n, (a->topk + 4095) / 4096);
  n = std::min(n, steps);
  const int per = (steps + n - 1) / n;
  pl.split_keys = per * 32;
  pl.n = (steps + per - 1) / per;
  const int64_t rows = (int64_t)a->Sq * a->Hq;
  const int64_t b = (int64_t)pl.n * rows * (a->d + 1) * 4;
  pl.bytes = b == 0 ? 0 : (b + 255) / 256 * 256;
  return pl;
}

}  // namespace

int64_t attn_sparse_fp8_workspace_bytes(const attn_sparse_fp8_args* a, int32_t n_splits) {
  g_last_error.clear();
  if (validate_fp8_shape(a) != ATTN_OK) return -1;
  if (n_splits < 0 || n_splits > kMaxSplits) {
    fail(ATTN_INVALID_ARGUMENT, "n_splits must be in [0, %d], got %d", kMaxSplits, n_splits);
    return -1;
  }
  return plan_fp8(a, n_splits).bytes;
}

attn_status attn_fwd_sparse_fp8(const attn_sparse_fp8_args* a, int32_t n_splits, void* workspace,
                                int64_t workspace_bytes, void* stream) {
  g_last_error.clear();
  attn_status st = validate_fp8_shape(a);
  if (st != ATTN_OK) return st;
  if (n_splits < 0 || n_splits > kMaxSplits)
    return fail(ATTN_INVALID_ARGUMENT, "n_splits must be in [0, %d], got %d", kMaxSplits, n_splits);
  if (a->Sq == 0) return ATTN_OK;
  if (!a->q || !a->codes || !a->scales || !a->out || !a->lse || (a->topk > 0 && !a->indices))
    return fail(ATTN_INVALID_ARGUMENT, "q, codes, scales, out, lse (and indices when topk > 0) must be non-NULL");
  if (!aligned16(a->q) || !aligned16(a->codes) || !aligned16(a->scales) || !aligned16(a->out) ||
      !aligned16(a->lse) || !aligned16(a->sinks) || ((uintptr_t)a->indices & 3u))
    return fail(ATTN_INVALID_ARGUMENT, "device pointers must be 16-byte aligned (indices 4-byte)");
  if (a->q_ss < 0 || a->q_sh < 0 || a->o_ss < 0 || a->o_sh < 0 || ((a->q_ss | a->q_sh | a->o_ss | a->o_sh) & 7))
    return fail(ATTN_INVALID_ARGUMENT, "q and out strides must be >= 0 and multiples of 8 elements");
  if (a->c_sn < a->d || (a->c_sn & 15) || a->s_sn < a->d / 128 || (a->s_sn & 3))
    return fail(ATTN_INVALID_ARGUMENT, "code rows need >= d bytes (multiple of 16), scale rows >= d/128 floats (multiple of 4)");
  if ((int64_t)a->N * a->c_sn >= ((int64_t)1 << 32) || (int64_t)a->N * a->s_sn * 4 >= ((int64_t)1 << 32))
    return fail(ATTN_INVALID_ARGUMENT, "the pool must stay below 4 GiB of codes and of scales");
  if (a->topk > 0 && a->idx_ss < a->topk) return fail(ATTN_INVALID_ARGUMENT, "index row stride smaller than topk");
  const Fp8Plan pl = plan_fp8(a, n_splits);
  if (pl.bytes > 0 && (workspace == nullptr || workspace_bytes < pl.bytes))
    return fail(ATTN_INVALID_ARGUMENT, "the fp8 sparse decode needs a workspace of %lld bytes, got %lld",
                (long long)pl.bytes, (long long)(workspace ? workspace_bytes : 0));
  if (!aligned16(workspace)) return fail(ATTN_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  const int64_t rows = (int64_t)a->Sq * a->Hq;
  attn::SpFp8Params p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.codes = a->codes; p.scales = a->scales; p.idx = a->indices;
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = p.part_o + (int64_t)pl.n * rows * a->d;
  p.q_ss = a->q_ss; p.q_sh = a->q_sh; p.c_sn = a->c_sn; p.s_sn = a->s_sn; p.idx_ss = a->idx_ss;
  p.Sq = a->Sq; p.Hq = a->Hq; p.N = a->N; p.topk = a->topk; p.split_keys = pl.split_keys; p.n_splits = pl.n;
  p.scale = a->scale;
  p.c = a->scale * 1.4426950408889634f;
  int err = attn::launch_sparse_fp8(p, stream);
  if (err != 0) return fail(ATTN_HIP_ERROR, "launch of the fp8 sparse decode failed: %s", hipGetErrorString((hipError_t)err));
  attn::MergeParams m;
  std::memset(&m, 0, sizeof(m));
  m.part_o = p.part_o; m.part_lse = p.part_lse; m.sinks = a->sinks; m.out = a->out; m.lse = a->lse;
  m.o_sb = a->o_ss; m.o_sh = a->o_sh; m.o_st = 0;
  m.B = a->Sq; m.H = a->Hq; m.Tq = 1; m.n_splits = pl.n; m.d_v = a->d; m.f32 = 0;
  err = attn::launch_merge(m, stream);
  if (err != 0) return fail(ATTN_HIP_ERROR, "launch of the merge failed: %s", hipGetErrorString((hipError_t)err));
  note_dispatch(kFp8Slot, kFp8Path);
  note_dispatch(kMergeSlot, kMergePath);
  return ATTN_OK;
}

// ---------------------------------------------------------------- sparse top-k backward
namespace {

static attn_status validate_sparse_bwd_shape(const attn_sparse_bwd_args* a) {
  if (!a) return fail(ATTN_INVALID_ARGUMENT, "args is NULL");
  if (a->struct_size != sizeof(attn_sparse_bwd_args))
    return fail(ATTN_ABI_MISMATCH, "attn_sparse_bwd_args.struct_size = %u, library expects %zu", a->struct_size,
                sizeof(attn_sparse_bwd_args));
  if (a->dtype != ATTN_BF16) return fail(ATTN_UNSUPPORTED, "the sparse backward is compiled for bf16 only");
  if (a->Sq < 0 || a->Hq < 1 || a->N < 1 || a->topk < 0) return fail(ATTN_INVALID_ARGUMENT, "bad Sq/Hq/N/topk");
  if (a->d_qk != 512 || a->d_v != 512 || a->Hq != 64)
    return fail(ATTN_UNSUPPORTED, "the sparse backward is compiled for d_qk = d_v = 512 and Hq = 64 (got %d, %d, %d)",
                a->d_qk, a->d_v, a->Hq);
  if (!(std::isfinite(a->scale) && a->scale > 0.f)) return fail(ATTN_INVALID_ARGUMENT, "scale must be finite and > 0");
  return ATTN_OK;
}

static int64_t sparse_bwd_workspace(const attn_sparse_bwd_args* a) {
  const int64_t b = (int64_t)a->Sq * a->Hq * 4;
  return b == 0 ? 0 : (b + 255) / 256 * 256;
}

}  // namespace

int64_t attn_bwd_sparse_workspace_bytes(const attn_sparse_bwd_args* a) {
  g_last_error.clear();
  if (validate_sparse_bwd_shape(a) != ATTN_OK) return -1;
  return sparse_bwd_workspace(a);
}

attn_status attn_bwd_sparse_topk(const attn_sparse_bwd_args* a, void* workspace, int64_t workspace_bytes,
                                 void* stream) {
  g_last_error.clear();
  attn_status st = validate_sparse_bwd_shape(a);
  if (st != ATTN_OK) return st;
  if (!a->kv || !a->dkv) return fail(ATTN_INVALID_ARGUMENT, "kv and dkv must be non-NULL");
  if (a->Sq > 0 && (!a->q || !a->out || !a->dout || !a->lse || !a->dq || (a->topk > 0 && !a->indices)))
    return fail(ATTN_INVALID_ARGUMENT, "q, out, dout, lse, dq (and indices when topk > 0) must be non-NULL");
  if (a->dsinks && !a->sinks) return fail(ATTN_INVALID_ARGUMENT, "dsinks needs sinks");
  if (!aligned16(a->q) || !aligned16(a->kv) || !aligned16(a->out) || !aligned16(a->dout) || !aligned16(a->lse) ||
      !aligned16(a->dq) || !aligned16(a->dkv) || ((uintptr_t)a->indices & 3u) || !aligned16(a->sinks) ||
      ((uintptr_t)a->dsinks & 3u))
    return fail(ATTN_INVALID_ARGUMENT, "device pointers must be 16-byte aligned (indices, dsinks 4-byte)");
  const int64_t strides[] = {a->q_ss, a->q_sh, a->kv_sn, a->o_ss, a->o_sh, a->do_ss, a->do_sh, a->dq_ss, a->dq_sh};
  for (int64_t x : strides)
    if (x < 0 || x % 8 != 0)
      return fail(ATTN_INVALID_ARGUMENT, "strides must be >= 0 and multiples of 8 elements");
  if (a->kv_sn < a->d_qk) return fail(ATTN_INVALID_ARGUMENT, "kv row stride smaller than d_qk");
  if (a->dkv_sn < a->d_qk || a->dkv_sn % 4 != 0)
    return fail(ATTN_INVALID_ARGUMENT, "dkv row stride must be >= d_qk and a multiple of 4");
  if (a->idx_ss < a->topk) return fail(ATTN_INVALID_ARGUMENT, "index row stride smaller than topk");
  const int64_t need = sparse_bwd_workspace(a);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(ATTN_INVALID_ARGUMENT, "the sparse backward needs a workspace of %lld bytes, got %lld",
                (long long)need, (long long)(workspace ? workspace_bytes : 0));
  if (!aligned16(workspace)) return fail(ATTN_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  attn::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = a->kv; p.v = a->kv; p.out = a->out; p.dout = a->dout; p.lse = a->lse; p.sinks = a->sinks;
  p.dq = a->dq; p.dsinks = a->dsinks;
  p.D = static_cast<float*>(workspace);
  p.q_sb = a->q_ss; p.q_sh = a->q_sh;
  p.k_st = a->kv_sn; p.v_st = a->kv_sn;
  p.o_sb = a->o_ss; p.o_sh = a->o_sh;
  p.do_sb = a->do_ss; p.do_sh = a->do_sh;
  p.dq_sb = a->dq_ss; p.dq_sh = a->dq_sh;
  p.B = a->Sq; p.H = a->Hq; p.Hkv = 1; p.Tq = 1; p.Tk = a->topk; p.g = a->Hq;
  p.scale = a->scale;
  p.c = a->scale * 1.4426950408889634f;
  p.idx = a->indices; p.idx_ss = a->idx_ss;
  p.npool = a->N; p.topk = a->topk;
  p.dkv = a->dkv; p.dkv_sn = a->dkv_sn;
  const int err = attn::launch_bwd_sparse(p, stream);
  if (err != 0)
    return fail(ATTN_HIP_ERROR, "launch of the sparse backward failed: %s", hipGetErrorString((hipError_t)err));
  note_dispatch(kSpBwdSlot, kSpBwdPath);
  return ATTN_OK;
}

// ---------------------------------------------------------------- quantized K/V decode
namespace {

// index into kQkvPaths: (q8_0, q4_0) x (d 128, d 256, d 512)
static int qkv_path(int fmt, int d) {
  const int f = fmt == ATTN_KV_Q8_0 ? 0 : (fmt == ATTN_KV_Q4_0 ? 1 : -1);
  if (f < 0 || (d != 128 && d != 256 && d != 512)) return -1;
  return f + (d == 256 ? 2 : (d == 512 ? 4 : 0));
}

static attn_status validate_qkv_shape(const attn_qkv_args* a) {
  if (!a) return fail(ATTN_INVALID_ARGUMENT, "args is NULL");
  if (a->struct_size != sizeof(attn_qkv_args))
    return fail(ATTN_ABI_MISMATCH, "attn_qkv_args.struct_size = %u, library expects %zu", a->struct_size,
                sizeof(attn_qkv_args));
  if (a->kv_format != ATTN_KV_Q8_0 && a->kv_format != ATTN_KV_Q4_0)
    return fail(ATTN_UNSUPPORTED, "kv_format %d unsupported (q8_0 = 8, q4_0 = 2)", a->kv_format);
  if (a->B < 1 || a->H < 1 || a->Hkv < 1) return fail(ATTN_INVALID_ARGUMENT, "B, H, Hkv must be >= 1");
  if (a->Tq < 0 || a->Tk < 0) return fail(ATTN_INVALID_ARGUMENT, "Tq, Tk must be >= 0");
  if (a->H % a->Hkv != 0) return fail(ATTN_INVALID_ARGUMENT, "H (%d) must be a multiple of Hkv (%d)", a->H, a->Hkv);
  if (!(std::isfinite(a->scale) && a->scale > 0.f)) return fail(ATTN_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (a->causal != 0 && a->causal != 1) return fail(ATTN_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (qkv_path(a->kv_format, a->d) < 0) return fail(ATTN_UNSUPPORTED, "no compiled quantized-cache kernel for d = %d", a->d);
  return ATTN_OK;
}

static int64_t qkv_row_bytes(const attn_qkv_args* a) { return (int64_t)a->d / 32 * (a->kv_format == ATTN_KV_Q8_0 ? 34 : 18); }

static attn_status validate_qkv(const attn_qkv_args* a) {
  const attn_status s = validate_qkv_shape(a);
  if (s != ATTN_OK) return s;
  if (a->Tq > 0 && (!a->q || !a->out || !a->lse)) return fail(ATTN_INVALID_ARGUMENT, "q, out, lse must be non-NULL");
  if (a->Tk > 0 && (!a->k || !a->v)) return fail(ATTN_INVALID_ARGUMENT, "k, v must be non-NULL when Tk > 0");
  if (!aligned16(a->q) || !aligned16(a->out) || !aligned16(a->lse) || !aligned16(a->sinks))
    return fail(ATTN_INVALID_ARGUMENT, "q, out, lse, sinks must be 16-byte aligned");
  if (((uintptr_t)a->k | (uintptr_t)a->v) & 3u) return fail(ATTN_INVALID_ARGUMENT, "k, v must be 4-byte aligned");
  const int64_t es[] = {a->q_sb, a->q_sh, a->q_st, a->o_sb, a->o_sh, a->o_st};
  for (int64_t x : es)
    if (x < 0 || x % 8 != 0) return fail(ATTN_INVALID_ARGUMENT, "q/out strides must be >= 0 multiples of 8 elements");
  const int64_t bs[] = {a->k_sb, a->k_sh, a->k_st, a->v_sb, a->v_sh, a->v_st};
  for (int64_t x : bs)
    if (x < 0 || x % 4 != 0) return fail(ATTN_INVALID_ARGUMENT, "k/v byte strides must be >= 0 multiples of 4");
  if (a->Tk > 1 && (a->k_st < qkv_row_bytes(a) || a->v_st < qkv_row_bytes(a)))
    return fail(ATTN_INVALID_ARGUMENT, "k/v token stride smaller than a row (%lld bytes)", (long long)qkv_row_bytes(a));
  if (a->Tq > 1 && (a->q_st < a->d || a->o_st < a->d))
    return fail(ATTN_INVALID_ARGUMENT, "q/out token stride smaller than d");
  if ((int64_t)a->Tk * std::max(a->k_st, a->v_st) >= ((int64_t)1 << 31))
    return fail(ATTN_INVALID_ARGUMENT, "k/v of one head must span less than 2^31 bytes");
  return ATTN_OK;
}

struct QkvPlan {
  int n, keys, n_rt, rt;
  int64_t bytes;
};

static QkvPlan plan_qkv(const attn_qkv_args* a, int n_req) {
  // a workgroup owns 16 rt folded query rows of one (b, kv head)
  const int64_t rows = (int64_t)(a->H / a->Hkv) * a->Tq;
  const int rt = attn::qkv_row_tiles(a->kv_format, a->d, (int)std::min<int64_t>(rows, 1 << 30));
  QkvPlan pl{1, a->Tk, (int)((rows + 16 * rt - 1) / (16 * rt)), rt, 0};
  const int nblocks = (a->Tk + 31) / 32;
  if (nblocks <= 1 || a->Tq == 0) return pl;
  int want = n_req;
  if (want == 0) {
    int occ = attn::occupancy_qkv(a->kv_format, a->d, pl.rt);
    if (occ <= 0) occ = 4;
    const int64_t tiles = (int64_t)pl.n_rt * a->B * a->Hkv;
    want = (int)std::min<int64_t>(kMaxSplits, std::max<int64_t>(1, (int64_t)device_cus() * occ / tiles));
  }
  want = std::min(want, nblocks);
  if (want <= 1) return pl;
  const int per = (nblocks + want - 1) / want;
  pl.keys = per * 32;
  pl.n = (a->Tk + pl.keys - 1) / pl.keys;
  if (pl.n <= 1) {
    pl.n = 1;
    pl.keys = a->Tk;
    return pl;
  }
  pl.bytes = (int64_t)pl.n * a->B * a->H * a->Tq * ((int64_t)a->d + 1) * 4;
  return pl;
}

}  // namespace

int64_t attn_qkv_workspace_bytes(const attn_qkv_args* a, int32_t n_splits) {
  g_last_error.clear();
  if (validate_qkv_shape(a) != ATTN_OK) return -1;
  if (n_splits < 0 || n_splits > kMaxSplits) {
    fail(ATTN_INVALID_ARGUMENT, "n_splits must be in [0, %d], got %d", kMaxSplits, n_splits);
    return -1;
  }
  return plan_qkv(a, n_splits).bytes;
}

attn_status attn_fwd_dense_qkv(const attn_qkv_args* a, int32_t n_splits, void* workspace, int64_t workspace_bytes,
                               void* stream) {
  g_last_error.clear();
  attn_status s = validate_qkv(a);
  if (s != ATTN_OK) return s;
  if (n_splits < 0 || n_splits > kMaxSplits)
    return fail(ATTN_INVALID_ARGUMENT, "n_splits must be in [0, %d], got %d", kMaxSplits, n_splits);
  if (a->Tq == 0) return ATTN_OK;
  const QkvPlan pl = plan_qkv(a, n_splits);
  if (pl.n > 1) {
    if (workspace == nullptr || workspace_bytes < pl.bytes)
      return fail(ATTN_INVALID_ARGUMENT, "%d key ranges need a workspace of %lld bytes, got %lld", pl.n,
                  (long long)pl.bytes, (long long)(workspace ? workspace_bytes : 0));
    if (!aligned16(workspace)) return fail(ATTN_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  }
  attn::QkvParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = static_cast<const unsigned char*>(a->k); p.v = static_cast<const unsigned char*>(a->v);
  p.out = a->out; p.lse = a->lse; p.sinks = a->sinks;
  p.q_sb = a->q_sb; p.q_sh = a->q_sh; p.q_st = a->q_st;
  p.k_sb = a->k_sb; p.k_sh = a->k_sh; p.k_st = a->k_st;
  p.v_sb = a->v_sb; p.v_sh = a->v_sh; p.v_st = a->v_st;
  p.o_sb = a->o_sb; p.o_sh = a->o_sh; p.o_st = a->o_st;
  p.B = a->B; p.H = a->H; p.Hkv = a->Hkv; p.Tq = a->Tq; p.Tk = a->Tk; p.g = a->H / a->Hkv;
  p.causal = a->causal;
  p.scale = a->scale;
  p.c = a->scale * 1.4426950408889634f;
  p.n_rt = pl.n_rt;
  p.n_splits = pl.n;
  p.split_keys = pl.keys;
  if (pl.n > 1) {
    p.part_o = static_cast<float*>(workspace);
    p.part_lse = p.part_o + (int64_t)pl.n * a->B * a->H * a->Tq * a->d;
  }
  int err = attn::launch_qkv(p, a->kv_format, a->d, pl.rt, stream);
  if (err != 0)
    return fail(ATTN_HIP_ERROR, "launch of the quantized-cache kernel failed: %s", hipGetErrorString((hipError_t)err));
  const int qp = qkv_path(a->kv_format, a->d);
  note_dispatch(kQkvSlot0 + qp, kQkvPaths[qp]);
  if (pl.n > 1) {
    attn::MergeParams m;
    std::memset(&m, 0, sizeof(m));
    m.part_o = p.part_o; m.part_lse = p.part_lse; m.sinks = a->sinks; m.out = a->out; m.lse = a->lse;
    m.o_sb = a->o_sb; m.o_sh = a->o_sh; m.o_st = a->o_st;
    m.B = a->B; m.H = a->H; m.Tq = a->Tq; m.d_v = a->d; m.n_splits = pl.n; m.f32 = 0;
    err = attn::launch_merge(m, stream);
    if (err != 0) return fail(ATTN_HIP_ERROR, "launch of the split merge failed: %s", hipGetErrorString((hipError_t)err));
    note_dispatch(kMergeSlot, kMergePath);
  }
  return ATTN_OK;
}

// ---------------------------------------------------------------- packed variable-length batches
attn_status attn_fwd_varlen(const attn_varlen_args* a, void* stream) {
  g_last_error.clear();
  if (!a) return fail(ATTN_INVALID_ARGUMENT, "args is NULL");
  if (a->struct_size != sizeof(attn_varlen_args))
    return fail(ATTN_ABI_MISMATCH, "attn_varlen_args.struct_size = %u, library expects %zu", a->struct_size,
                sizeof(attn_varlen_args));
  if (a->dtype != ATTN_BF16) return fail(ATTN_UNSUPPORTED, "packed batches are compiled for bf16 only");
  if (a->B < 1 || a->max_seqlen_q < 0 || a->total_q < 0 || a->total_k < 0)
    return fail(ATTN_INVALID_ARGUMENT, "B >= 1 and max_seqlen_q, total_q, total_k >= 0 required");
  if (a->total_q > 0 && (!a->cu_seqlens_q || !a->cu_seqlens_k))
    return fail(ATTN_INVALID_ARGUMENT, "cu_seqlens_q and cu_seqlens_k must be non-NULL");
  if (((uintptr_t)a->cu_seqlens_q | (uintptr_t)a->cu_seqlens_k) & 3u)
    return fail(ATTN_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  // the dense validation on an equivalent strided view: B sequences of
  // max_seqlen_q queries (batch strides 0) and up to total_k keys
  attn_dense_args d;
  std::memset(&d, 0, sizeof(d));
  d.struct_size = sizeof(d);
  d.dtype = a->dtype;
  d.B = a->B; d.H = a->H; d.Hkv = a->Hkv; d.Tq = a->max_seqlen_q; d.Tk = a->total_k;
  d.d_qk = a->d_qk; d.d_v = a->d_v; d.causal = a->causal; d.scale = a->scale;
  d.q = a->q; d.q_sb = 0; d.q_sh = a->q_sh; d.q_st = a->q_st;
  d.k = a->k; d.k_sb = 0; d.k_sh = a->k_sh; d.k_st = a->k_st;
  d.v = a->v; d.v_sb = 0; d.v_sh = a->v_sh; d.v_st = a->v_st;
  d.out = a->out; d.o_sb = 0; d.o_sh = a->o_sh; d.o_st = a->o_st;
  d.lse = a->lse; d.sinks = a->sinks;
  d.window_left = a->window_left; d.window_right = a->window_right;
  DensePlan dp;
  attn_status s = validate_dense(&d, &dp);
  if (s != ATTN_OK) return s;
  if (dp.cfg->dtype != 0 || a->d_qk > 256)
    return fail(ATTN_UNSUPPORTED, "no packed-batch kernel for these head dims (bf16, d_qk <= 256)");
  if (a->total_q == 0 || a->max_seqlen_q == 0) return ATTN_OK;
  attn::KernelParams& p = dp.kp;
  const int BM = dp.cfg->block_rows;
  p.varlen = 1;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.total_q = a->total_q;
  p.total_k = a->total_k;
  p.fold_tm = 1;
  p.aligned = 0;
  p.tiles_per_head = 0;
  const int64_t tpg = ((int64_t)p.g * a->max_seqlen_q + BM - 1) / BM;
  const int64_t tiles = (int64_t)p.n_groups * tpg;
  if (tiles > 0x7fffffff) return fail(ATTN_INVALID_ARGUMENT, "problem too large for one launch");
  p.tiles_per_group = (int)tpg;
  p.n_tiles = (int)tiles;
  plan_xcd(p, 2);
  return do_launch(dp, stream);
}

uint64_t attn_dispatch_count(const char* path) {
  if (!path) return 0;
  const int i = path_index(path);
  return i < 0 ? 0 : g_counts[i].load(std::memory_order_relaxed);
}

void attn_reset_dispatch_counts(void) {
  for (int i = 0; i < kMaxPaths; ++i) g_counts[i].store(0, std::memory_order_relaxed);
}

int64_t attn_budget_tile_rows(int64_t budget_bytes, int64_t Tk, int64_t elt_bytes) {
  if (budget_bytes <= 0 || Tk <= 0 || elt_bytes <= 0) return 0;
  const int64_t r = budget_bytes / (Tk * elt_bytes);
  return r > 0 ? r : 1;
}

}  // extern "C"
