// Attention backward (and the kernels that share its tiling) for AMD CDNA4
// (gfx950 / MI355X), bf16 inputs.
//
// Gradients of O = softmax(scale * Q K^T + mask [+ sink in the denominator]) V
// with respect to q, k, v and the sinks, from the forward's inputs, its
// output O and lse, and dO = dL/dO. This is the raw attention backward that
// follows the forward and the output merge in TransformerEngine's
// context-parallel attention ("Flowchart": raw backward -> Q/K/V gradients;
// "Summary": raw forward/backward wrappers with LSE handling). With
// P = exp(scale * q.k - lse) recomputed from the saved lse:
//
//   D    = rowsum(dO * O)                       (row dots)
//   dV   = P^T dO,  dP = dO V^T,  dS = P (dP - D)
//   dK   = scale dS^T Q,  dQ = scale dS K
//   dsink_h = -sum over rows of exp(sink_h - lse) D
//
// GQA/MQA: the keys of kv head kvh are read by the g query heads kvh*g ..
// kvh*g + g-1 (kv-major), so dK and dV sum over those heads.
//
// Four launches (five with a head split), none with atomics (the result does
// not depend on timing):
//
//  1. bwd_dot_kernel   D for every row, several rows per wave.
//  2. bwd_dsink_kernel one workgroup per head sums its rows' sink terms.
//  3. bwd_dkdv_kernel  a workgroup owns 32 keys per wave of one (b, kv head);
//                      K and V of its keys stay in registers (the B operands
//                      of S = Q K^T and dP = dO V^T) while it streams the
//                      query rows of all g heads through LDS (Q and dO tiles);
//                      dV^T += dO^T P and dK^T += Q^T dS take their A operands
//                      from the same tiles by transposed LDS reads and their
//                      B operands straight from the P / dS accumulators.
//  4. bwd_dq_kernel    a workgroup owns 32 folded query rows per wave (the
//                      forward's tiling); Q and dO rows stay in registers
//                      while K and V blocks stream through LDS; S^T and dP^T
//                      are recomputed and dQ^T += K^T dS^T.
//
// (Steps 3 and 4 for 64/128-wide heads: bwd_dkdv_pair_kernel, K and V in LDS
// and two waves per SIMD; for 256/512-wide heads: bwd_dkdv_wide_kernel and
// bwd_dq_wide_kernel, the columns split over waves whose partial products
// meet in LDS, see section 4b.)
//
// Scores and probabilities never leave the CU; the workspace holds D and, for
// 256/512-wide heads with few key blocks, fp32 dK/dV partials of head splits
// that a fifth kernel (bwd_wide_reduce_kernel) adds in a fixed order.
//
// The file also holds the kernels built on the same tile helpers (row and
// transposed fragment reads, DMA tile loads):
//
//  5. bwd_sparse_kernel   the sparse top-k backward (pool gradient by fp32
//                         atomics), after a fill, the row dots and the sinks.
//  6. extras_kernel       the forward's extra returns (probabilities, row
//                         maxima) as a second pass from q, k and lse.
//  7. fwd_dropout_kernel  the forward with a caller-drawn dropout mask, heads
//                         up to 256 wide (512-wide heads take the mask inside
//                         the fused forward); the backward kernels above take
//                         the same mask.
//  8. sparse_fp8_kernel   the sparse top-k decode over an fp8 pool.

#include <hip/hip_runtime.h>
#include <algorithm>
#include <stdint.h>

#include "attn_params.h"

namespace attn {
namespace {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// two floats -> two bf16 (round to nearest even)
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  const u32x4 w = {pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, w);
}

// bf16 halves of a 32-bit word, widened exactly
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16-byte chunk swizzle of a tile row with CPR chunks (64 LDS banks): 16
// consecutive rows send one logical chunk to distinct bank groups, and
// aligned groups of 4 rows send a 4-chunk group to distinct groups. Rows of
// 128 + 256n bytes use a 3-bit XOR inside aligned 8-chunk groups.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  static_assert(CPR % 8 == 0, "rows are whole 8-chunk groups");
  if constexpr (CPR % 16 == 0)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// element offset of logical chunk c of tile row r
template <int CPR>
__device__ __forceinline__ int chunk_at(int r, int c) {
  return r * (CPR * 8) + ((c ^ swz<CPR>(r)) << 3);
}

// A operand (rows of a row-major tile): lane row `row`, columns 16s + 8lh .. +7
template <int CPR>
__device__ __forceinline__ bf16x8 row_frag(const bf16_t* tile, int row, int s, int lh) {
  return *reinterpret_cast<const bf16x8*>(tile + chunk_at<CPR>(row, 2 * s + lh));
}

// A operand X^T (32 columns of X by 16 rows) from a row-major tile X by two
// transposed reads. The 16 rows r0..r0+15 (r0 a multiple of 16) arrive in the
// order {0-3, 8-11} for lanes 0-31 and {4-7, 12-15} for lanes 32-63, which is
// the order in which a 32x32 accumulator with those rows hands them to the B
// operand (pack8 of its elements 8ks..8ks+7), so no shuffle is needed.
template <int CPR>
__device__ __forceinline__ bf16x8 tr_frag(const bf16_t* tile, int r0, int c0, int lane) {
  const int vg = lane >> 4, vi = lane & 15;
  const int vrow = (vg >> 1) * 4 + (vi >> 2);
  const int col = c0 + (vg & 1) * 16 + 4 * (vi & 3);
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = r0 + vrow + 8 * h;
    const bf16_t* ptr = tile + row * (CPR * 8) + (((col >> 3) ^ swz<CPR>(row)) << 3) + (col & 7);
    const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)ptr);
    w[2 * h] = (uint32_t)(uint16_t)t[0] | ((uint32_t)(uint16_t)t[1] << 16);
    w[2 * h + 1] = (uint32_t)(uint16_t)t[2] | ((uint32_t)(uint16_t)t[3] << 16);
  }
  return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
}

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O): LPR = DV/8 lanes per row, 64/LPR rows per wave
// ---------------------------------------------------------------------------
template <int DV>
__global__ void __launch_bounds__(256) bwd_dot_kernel(const BwdParams p) {
  constexpr int LPR = DV / 8, RPW = 64 / LPR;
  static_assert(LPR <= 64 && (LPR & (LPR - 1)) == 0, "power-of-two lanes per row");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t R = (int64_t)p.B * p.H * p.Tq;
  const int64_t row = ((int64_t)blockIdx.x * 4 + wave) * RPW + lane / LPR;
  const int c = lane % LPR;
  float s = 0.f;
  if (row < R) {
    const int t = (int)(row % p.Tq);
    const int h = (int)((row / p.Tq) % p.H);
    const int b = (int)(row / ((int64_t)p.Tq * p.H));
    const u32x4 o = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(p.out) + b * p.o_sb +
                                                    h * p.o_sh + t * p.o_st + c * 8);
    const u32x4 d = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(p.dout) + b * p.do_sb +
                                                    h * p.do_sh + t * p.do_st + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) s += bf_lo(o[e]) * bf_lo(d[e]) + bf_hi(o[e]) * bf_hi(d[e]);
  }
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if (row < R && c == 0) p.D[row] = s;
}

// ---------------------------------------------------------------------------
// 2. dsink_h = -sum_{b,t} exp(sink_h - lse) D
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_dsink_kernel(const BwdParams p) {
  __shared__ float part[4];
  const int h = blockIdx.x;
  const float sk = p.sinks[h];
  float s = 0.f;
  const int n = p.B * p.Tq;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int b = i / p.Tq, t = i % p.Tq;
    const int64_t row = ((int64_t)b * p.H + h) * p.Tq + t;
    const float l = p.lse[row];
    if (l != -INFINITY && sk != -INFINITY) s += __expf(sk - l) * p.D[row];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) p.dsinks[h] = -((part[0] + part[1]) + (part[2] + part[3]));
}

// ---------------------------------------------------------------------------
// Tile loads: global_load_lds moves 16 (or 4) bytes per lane from global
// memory straight into LDS at m0 + lane * size, from a wave-uniform base in
// scalar registers plus a per-lane 32-bit byte offset. The waits are explicit
// (vmcnt), since the compiler does not see these loads.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lds_u32(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ptr;
}

__device__ __forceinline__ const void* uniform_ptr(const void* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

__device__ __forceinline__ void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// vmcnt wait with a wave-uniform count (0..7)
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
  }
}
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kPF = 2;  // LDS operand reads kept ahead of the MFMAs (2 measured best)

// N MFMAs each fed by R LDS reads: keep PF MFMAs' reads in flight ahead
template <int N, int R>
__device__ __forceinline__ void pipeline_reads() {
  constexpr int PD = N < kPF ? N : kPF;
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, R * PD, 0);
#pragma unroll
  for (int k = 0; k < N - PD; ++k) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, PD, 0);
}

// DMA of BR rows (starting at row r0 of a row-major source with element row
// stride `st`, rows past `rmax` clamped onto it) into a swizzled LDS tile of
// CPR chunks per row: wave instruction j fills LDS slots 64j .. 64j+63, and
// slot (r, c') receives logical chunk c' ^ swz(r) of row r.
template <int CPR, int BR, int NW>
__device__ __forceinline__ void dma_tile(const bf16_t* base, int64_t st, int r0, int rmax, uint32_t lds, int wave,
                                         int lane) {
  constexpr int NI = BR * CPR / 64;
  static_assert(BR * CPR % 64 == 0, "whole wave instructions");
  const void* sb = uniform_ptr(base + (int64_t)r0 * st);
#pragma unroll
  for (int m = 0; m < (NI + NW - 1) / NW; ++m) {
    const int j = wave + NW * m;
    if (NI % NW != 0 && j >= NI) break;
    const int sl = 64 * j + lane, r = sl / CPR, c = (sl % CPR) ^ swz<CPR>(sl / CPR);
    const int rr = min(r0 + r, rmax) - r0;
    dma16(sb, 2u * (uint32_t)(rr * (int32_t)st + c * 8), lds + 1024u * j);
  }
}

// ---------------------------------------------------------------------------
// 3. dK, dV: one workgroup per 32*NW keys of one (b, kv head)
// ---------------------------------------------------------------------------
template <int DQK, int DV, int NW, int BQ, bool DROP>
__global__ void __launch_bounds__(NW * 64) bwd_dkdv_kernel(const BwdParams p) {
  constexpr int BNK = 32 * NW;  // keys per workgroup; BQ query rows per step (32-row sub-blocks)
  constexpr int CPQ = DQK / 8, CPO = DV / 8;
  constexpr int KS = DQK / 16, VS = DV / 16, DTK = DQK / 32, DTV = DV / 32;
  constexpr int QT_BYTES = BQ * DQK * 2, OT_BYTES = BQ * DV * 2;
  // with dropout a stage also holds the keep words of its rows, one column of
  // 32 keys per wave: [wave][row]
  constexpr int MOFF = QT_BYTES + OT_BYTES + 2 * BQ * 4;
  constexpr int STAGE = MOFF + (DROP ? NW * BQ * 4 : 0);
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "head dims are whole 32-column tiles");
  static_assert(BQ <= 64, "one row statistic per lane");
  // two stages: [Q tile | dO tile | lse | D]
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, lh = lane >> 5;
  // key block 0 of every group first: under a causal mask the first key
  // blocks are seen by the most query rows
  const int n_groups = p.B * p.Hkv;
  const int grp = blockIdx.x % n_groups, b = grp / p.Hkv, kvh = grp % p.Hkv;
  const int kb0 = (blockIdx.x / n_groups) * BNK;
  const int key = kb0 + wave * 32 + lq;  // the key column this lane holds
  const int keyc = min(key, p.Tk - 1);

  bf16x8 kf[KS], vf[VS];
  {
    const bf16_t* kp = reinterpret_cast<const bf16_t*>(p.k) + b * p.k_sb + kvh * p.k_sh + (int64_t)keyc * p.k_st;
    const bf16_t* vp = reinterpret_cast<const bf16_t*>(p.v) + b * p.v_sb + kvh * p.v_sh + (int64_t)keyc * p.v_st;
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(kp + s * 16 + lh * 8);
#pragma unroll
    for (int s = 0; s < VS; ++s) vf[s] = *reinterpret_cast<const bf16x8*>(vp + s * 16 + lh * 8);
  }
  f32x16 ak[DTK], av[DTV];
#pragma unroll
  for (int dt = 0; dt < DTK; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) ak[dt][i] = 0.f;
#pragma unroll
  for (int dt = 0; dt < DTV; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) av[dt][i] = 0.f;

  const int off = p.Tk - p.Tq;
  // keys after its diagonal position a row may see (-1: unbounded); the
  // window never widens the causal bound
  const int up = p.causal ? 0 : p.win_right;
  // query tokens that can see a key of this block: from kb0 - off - up (the
  // upper bound) to kb0 + BNK - 1 - off + win_left (the window's lower bound)
  const int t_first = up >= 0 ? max(0, kb0 - off - up) : 0;
  const int t_last = p.win_left >= 0 ? min(p.Tq - 1, kb0 + BNK - 1 - off + p.win_left) : p.Tq - 1;
  const int ntb = (p.Tq + BQ - 1) / BQ;
  const int tb0 = min(t_first / BQ, ntb);
  const int per_head = t_last < t_first ? 0 : max(0, min(ntb, t_last / BQ + 1) - tb0);
  const int n_it = p.g * per_head;
  const uint32_t smem_s = lds_u32(smem);

  auto issue = [&](int it) {
    const int hl = it / per_head, t0 = (tb0 + it % per_head) * BQ;
    const int h = kvh * p.g + hl;
    const uint32_t st = smem_s + (uint32_t)((it & 1) * STAGE);
    dma_tile<CPQ, BQ, NW>(reinterpret_cast<const bf16_t*>(p.q) + b * p.q_sb + h * p.q_sh, p.q_st, t0, p.Tq - 1, st,
                          wave, lane);
    dma_tile<CPO, BQ, NW>(reinterpret_cast<const bf16_t*>(p.dout) + b * p.do_sb + h * p.do_sh, p.do_st, t0,
                          p.Tq - 1, st + QT_BYTES, wave, lane);
    if (wave == NW - 1) {
      // row statistics: lane l < BQ gets row t0 + l (clamped), 4 bytes each
      const int64_t rb = ((int64_t)b * p.H + h) * p.Tq + t0;
      const void* lb = uniform_ptr(p.lse + rb);
      const void* db = uniform_ptr(p.D + rb);
      const uint32_t vo = 4u * (uint32_t)(min(t0 + lane, p.Tq - 1) - t0);
      if (lane < BQ) {
        dma4(lb, vo, st + QT_BYTES + OT_BYTES);
        dma4(db, vo, st + QT_BYTES + OT_BYTES + BQ * 4);
      }
    }
    if constexpr (DROP) {
      // keep words of rows t0 .. t0+BQ-1 for this wave's 32 keys
      const int w = min(kb0 / 32 + wave, p.nwords - 1);
      const void* mb = uniform_ptr(p.keep + b * p.m_sb + h * p.m_sh + (int64_t)t0 * p.m_st + w);
      const uint32_t mo = 4u * (uint32_t)((min(t0 + lane, p.Tq - 1) - t0) * p.m_st);
      if (lane < BQ) dma4(mb, mo, st + MOFF + wave * BQ * 4);
    }
  };

  if (n_it > 0) issue(0);
  for (int it = 0; it < n_it; ++it) {
    wait_all_loads();  // this wave's loads of tile it have landed
    barrier();         // ... and everyone's; nobody reads the other stage any more
    if (it + 1 < n_it) issue(it + 1);
    const unsigned char* sp = smem + (it & 1) * STAGE;
    const bf16_t* qt = reinterpret_cast<const bf16_t*>(sp);
    const bf16_t* ot = reinterpret_cast<const bf16_t*>(sp + QT_BYTES);
    const float* rl = reinterpret_cast<const float*>(sp + QT_BYTES + OT_BYTES);
    const float* rd = rl + BQ;
    const int t0 = (tb0 + it % per_head) * BQ;
    // every (row, key) pair of the tile visible: no per-score mask
    const bool full = t0 + BQ <= p.Tq && kb0 + BNK <= p.Tk && (up < 0 || t0 + off + up >= kb0 + BNK - 1) &&
                      (p.win_left < 0 || t0 + BQ - 1 + off - p.win_left <= kb0);
#pragma unroll
    for (int qs = 0; qs < BQ / 32; ++qs) {
      f32x16 S, dP;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        S[i] = 0.f;
        dP[i] = 0.f;
      }
      const int r = qs * 32 + lq;
#pragma unroll
      for (int s = 0; s < (KS > VS ? KS : VS); ++s) {
        if (s < KS) S = mfma32(row_frag<CPQ>(qt, r, s, lh), kf[s], S);
        if (s < VS) dP = mfma32(row_frag<CPO>(ot, r, s, lh), vf[s], dP);
      }
      pipeline_reads<KS + VS, 1>();
      // accumulator element i holds query row qs*32 + lh*4 + 8*(i/4) + i%4 of key `key`
      float P[16], dS[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int r0 = qs * 32 + lh * 4 + 8 * g4;
        const f32x4 L = *reinterpret_cast<const f32x4*>(rl + r0);
        const f32x4 Dv = *reinterpret_cast<const f32x4*>(rd + r0);
        u32x4 M = {0u, 0u, 0u, 0u};
        if constexpr (DROP) M = *reinterpret_cast<const u32x4*>(rl + 2 * BQ + wave * BQ + r0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = g4 * 4 + j;
          float pr = __builtin_amdgcn_exp2f(fmaf(S[i], p.c, -L[j] * kLog2e));
          if (!full) {
            const int t = t0 + r0 + j;
            const int lim = t >= p.Tq ? -1 : (up >= 0 ? t + off + up : p.Tk - 1);
            const int lo = p.win_left >= 0 ? t + off - p.win_left : 0;
            pr = (key <= lim && key >= lo) ? pr : 0.f;
          }
          if constexpr (DROP) {
            // dV takes the dropped probabilities; dS = P (Z dP - D)
            const float z = ((M[j] >> lq) & 1u) ? p.inv_keep : 0.f;
            P[i] = pr * z;
            dS[i] = pr * (z * dP[i] - Dv[j]);
          } else {
            P[i] = pr;
            dS[i] = pr * (dP[i] - Dv[j]);
          }
        }
      }
      const bf16x8 pb0 = pack8(P), pb1 = pack8(P + 8);
      const bf16x8 db0 = pack8(dS), db1 = pack8(dS + 8);
#pragma unroll
      for (int dt = 0; dt < DTV; ++dt) {
        av[dt] = mfma32(tr_frag<CPO>(ot, qs * 32, dt * 32, lane), pb0, av[dt]);
        av[dt] = mfma32(tr_frag<CPO>(ot, qs * 32 + 16, dt * 32, lane), pb1, av[dt]);
      }
#pragma unroll
      for (int dt = 0; dt < DTK; ++dt) {
        ak[dt] = mfma32(tr_frag<CPQ>(qt, qs * 32, dt * 32, lane), db0, ak[dt]);
        ak[dt] = mfma32(tr_frag<CPQ>(qt, qs * 32 + 16, dt * 32, lane), db1, ak[dt]);
      }
      pipeline_reads<2 * (DTV + DTK), 2>();
    }
  }

  // dK^T / dV^T tiles: lane holds key `key`, columns dt*32 + 8*g4 + 4*lh .. +3
  if (key < p.Tk) {
    bf16_t* dkp = reinterpret_cast<bf16_t*>(p.dk) + b * p.dk_sb + kvh * p.dk_sh + (int64_t)key * p.dk_st;
    bf16_t* dvp = reinterpret_cast<bf16_t*>(p.dv) + b * p.dv_sb + kvh * p.dv_sh + (int64_t)key * p.dv_st;
#pragma unroll
    for (int dt = 0; dt < DTK; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + lh * 4;
        *reinterpret_cast<u32x2*>(dkp + d) = u32x2{pack2(ak[dt][g4 * 4] * p.scale, ak[dt][g4 * 4 + 1] * p.scale),
                                                   pack2(ak[dt][g4 * 4 + 2] * p.scale, ak[dt][g4 * 4 + 3] * p.scale)};
      }
#pragma unroll
    for (int dt = 0; dt < DTV; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + lh * 4;
        *reinterpret_cast<u32x2*>(dvp + d) =
            u32x2{pack2(av[dt][g4 * 4], av[dt][g4 * 4 + 1]), pack2(av[dt][g4 * 4 + 2], av[dt][g4 * 4 + 3])};
      }
  }
}

// ---------------------------------------------------------------------------
// 3b. dK, dV with two waves per SIMD (d_qk + d_v <= 256): eight waves own 128
// keys of one (b, kv head). Waves w and w+4 hold the same 32 keys and take
// the two 32-row halves of every 64-row query tile; K and V of the block sit
// in LDS for the whole kernel (the B operands of S and dP are read from there,
// which leaves the registers for the dK/dV accumulators), and the two partial
// sums of each key are added through LDS at the end.
// ---------------------------------------------------------------------------
template <int DQK, int DV, bool DROP>
__global__ void __launch_bounds__(512) bwd_dkdv_pair_kernel(const BwdParams p) {
  constexpr int NW = 8, BNK = 128, BQ = 64;
  constexpr int CPQ = DQK / 8, CPO = DV / 8;
  constexpr int KS = DQK / 16, VS = DV / 16, DTK = DQK / 32, DTV = DV / 32;
  constexpr int KT_BYTES = BNK * DQK * 2, VT_BYTES = BNK * DV * 2;
  constexpr int QT_BYTES = BQ * DQK * 2, OT_BYTES = BQ * DV * 2;
  // with dropout a stage also holds the keep words of its rows, one column of
  // 32 keys per key group: [cg][row]
  constexpr int MOFF = QT_BYTES + OT_BYTES + 2 * BQ * 4;
  constexpr int STAGE = MOFF + (DROP ? 4 * BQ * 4 : 0);
  constexpr int LDS_BYTES = KT_BYTES + VT_BYTES + 2 * STAGE;
  constexpr int RED_BYTES = 4 * (DTK + DTV) * 16 * 64 * 4;  // partial sums of waves 4..7
  static_assert(RED_BYTES <= LDS_BYTES && LDS_BYTES <= 160 * 1024, "LDS budget");
  // [K tile | V tile | stage 0 | stage 1], each stage [Q tile | dO tile | lse | D]
  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, lh = lane >> 5;
  const int cg = wave & 3, half = wave >> 2;  // key columns, query half
  const int n_groups = p.B * p.Hkv;
  // whole (b, kv head) groups on one XCD where the group count allows it
  // (workgroups are dealt to the 8 XCDs in turn), key block 0 of every
  // group first: under a causal mask the first key blocks see the most rows
  int grp_ = blockIdx.x % n_groups, kbi_ = blockIdx.x / n_groups;
  if (n_groups % 8 == 0) {
    const int slot = blockIdx.x / 8, gpx = n_groups / 8;
    grp_ = (blockIdx.x % 8) * gpx + slot % gpx;
    kbi_ = slot / gpx;
  }
  const int grp = grp_, b = grp / p.Hkv, kvh = grp % p.Hkv;
  const int kb0 = kbi_ * BNK;
  const int key = kb0 + cg * 32 + lq;
  const uint32_t smem_s = lds_u32(smem);
  const bf16_t* kt = reinterpret_cast<const bf16_t*>(smem);
  const bf16_t* vt = reinterpret_cast<const bf16_t*>(smem + KT_BYTES);

  f32x16 ak[DTK], av[DTV];
#pragma unroll
  for (int dt = 0; dt < DTK; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) ak[dt][i] = 0.f;
#pragma unroll
  for (int dt = 0; dt < DTV; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) av[dt][i] = 0.f;

  const int off = p.Tk - p.Tq;
  // keys after its diagonal position a row may see (-1: unbounded); the
  // window never widens the causal bound
  const int up = p.causal ? 0 : p.win_right;
  // query tokens that can see a key of this block: from kb0 - off - up (the
  // upper bound) to kb0 + BNK - 1 - off + win_left (the window's lower bound)
  const int t_first = up >= 0 ? max(0, kb0 - off - up) : 0;
  const int t_last = p.win_left >= 0 ? min(p.Tq - 1, kb0 + BNK - 1 - off + p.win_left) : p.Tq - 1;
  const int ntb = (p.Tq + BQ - 1) / BQ;
  const int tb0 = min(t_first / BQ, ntb);
  const int per_head = t_last < t_first ? 0 : max(0, min(ntb, t_last / BQ + 1) - tb0);
  const int n_it = p.g * per_head;
  // step it: query tile per_head-1-it/g (counted from tb0), head it%g of the
  // group; the tiles run downwards so that the workgroups of a group, which
  // share an XCD, read the same tile at about the same time (measured 1.5%)

  auto issue = [&](int it) {
    const int hl = it % p.g, t0 = (tb0 + per_head - 1 - it / p.g) * BQ;
    const int h = kvh * p.g + hl;
    const uint32_t st = smem_s + (uint32_t)(KT_BYTES + VT_BYTES + (it & 1) * STAGE);
    dma_tile<CPQ, BQ, NW>(reinterpret_cast<const bf16_t*>(p.q) + b * p.q_sb + h * p.q_sh, p.q_st, t0, p.Tq - 1, st,
                          wave, lane);
    dma_tile<CPO, BQ, NW>(reinterpret_cast<const bf16_t*>(p.dout) + b * p.do_sb + h * p.do_sh, p.do_st, t0,
                          p.Tq - 1, st + QT_BYTES, wave, lane);
    if (wave == NW - 1) {
      const int64_t rb = ((int64_t)b * p.H + h) * p.Tq + t0;
      const void* lb = uniform_ptr(p.lse + rb);
      const void* db = uniform_ptr(p.D + rb);
      const uint32_t vo = 4u * (uint32_t)(min(t0 + lane, p.Tq - 1) - t0);
      dma4(lb, vo, st + QT_BYTES + OT_BYTES);
      dma4(db, vo, st + QT_BYTES + OT_BYTES + BQ * 4);
    }
    if constexpr (DROP) {
      if (wave < 4) {
        // keep words of rows t0 .. t0+63 for key group `wave` (32 keys)
        const int w = min(kb0 / 32 + wave, p.nwords - 1);
        const void* mb = uniform_ptr(p.keep + b * p.m_sb + h * p.m_sh + (int64_t)t0 * p.m_st + w);
        const uint32_t mo = 4u * (uint32_t)((min(t0 + lane, p.Tq - 1) - t0) * p.m_st);
        dma4(mb, mo, st + MOFF + wave * BQ * 4);
      }
    }
  };

  // K and V of the block, once (rows past Tk clamped: they are masked)
  dma_tile<CPQ, BNK, NW>(reinterpret_cast<const bf16_t*>(p.k) + b * p.k_sb + kvh * p.k_sh, p.k_st, kb0, p.Tk - 1,
                         smem_s, wave, lane);
  dma_tile<CPO, BNK, NW>(reinterpret_cast<const bf16_t*>(p.v) + b * p.v_sb + kvh * p.v_sh, p.v_st, kb0, p.Tk - 1,
                         smem_s + KT_BYTES, wave, lane);
  if (n_it > 0) issue(0);
  for (int it = 0; it < n_it; ++it) {
    wait_all_loads();
    barrier();
    const unsigned char* sp = smem + KT_BYTES + VT_BYTES + (it & 1) * STAGE;
    const bf16_t* qt = reinterpret_cast<const bf16_t*>(sp);
    const bf16_t* ot = reinterpret_cast<const bf16_t*>(sp + QT_BYTES);
    const float* rl = reinterpret_cast<const float*>(sp + QT_BYTES + OT_BYTES);
    const float* rd = rl + BQ;
    const int t0 = (tb0 + per_head - 1 - it / p.g) * BQ;
    const bool full = t0 + BQ <= p.Tq && kb0 + BNK <= p.Tk && (up < 0 || t0 + off + up >= kb0 + BNK - 1) &&
                      (p.win_left < 0 || t0 + BQ - 1 + off - p.win_left <= kb0);
    const int qs = half;
    f32x16 S, dP;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      S[i] = 0.f;
      dP[i] = 0.f;
    }
    const int r = qs * 32 + lq, kr = cg * 32 + lq;
#pragma unroll
    for (int s = 0; s < (KS > VS ? KS : VS); ++s) {
      if (s < KS) S = mfma32(row_frag<CPQ>(qt, r, s, lh), row_frag<CPQ>(kt, kr, s, lh), S);
      if (s < VS) dP = mfma32(row_frag<CPO>(ot, r, s, lh), row_frag<CPO>(vt, kr, s, lh), dP);
    }
    pipeline_reads<KS + VS, 2>();
    // the next tile's loads go out once S and dP are formed (measured ~2%
    // faster than at the start of the step)
    if (it + 1 < n_it) issue(it + 1);
    float P[16], dS[16];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int r0 = qs * 32 + lh * 4 + 8 * g4;
      const f32x4 L = *reinterpret_cast<const f32x4*>(rl + r0);
      const f32x4 Dv = *reinterpret_cast<const f32x4*>(rd + r0);
      u32x4 M = {0u, 0u, 0u, 0u};
      if constexpr (DROP) M = *reinterpret_cast<const u32x4*>(rl + 2 * BQ + cg * BQ + r0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = g4 * 4 + j;
        float pr = __builtin_amdgcn_exp2f(fmaf(S[i], p.c, -L[j] * kLog2e));
        if (!full) {
          const int t = t0 + r0 + j;
          const int lim = t >= p.Tq ? -1 : (up >= 0 ? t + off + up : p.Tk - 1);
          const int lo = p.win_left >= 0 ? t + off - p.win_left : 0;
          pr = (key <= lim && key >= lo) ? pr : 0.f;
        }
        if constexpr (DROP) {
          const float z = ((M[j] >> lq) & 1u) ? p.inv_keep : 0.f;
          P[i] = pr * z;
          dS[i] = pr * (z * dP[i] - Dv[j]);
        } else {
          P[i] = pr;
          dS[i] = pr * (dP[i] - Dv[j]);
        }
      }
    }
    const bf16x8 pb0 = pack8(P), pb1 = pack8(P + 8);
    const bf16x8 db0 = pack8(dS), db1 = pack8(dS + 8);
#pragma unroll
    for (int dt = 0; dt < DTV; ++dt) {
      av[dt] = mfma32(tr_frag<CPO>(ot, qs * 32, dt * 32, lane), pb0, av[dt]);
      av[dt] = mfma32(tr_frag<CPO>(ot, qs * 32 + 16, dt * 32, lane), pb1, av[dt]);
    }
#pragma unroll
    for (int dt = 0; dt < DTK; ++dt) {
      ak[dt] = mfma32(tr_frag<CPQ>(qt, qs * 32, dt * 32, lane), db0, ak[dt]);
      ak[dt] = mfma32(tr_frag<CPQ>(qt, qs * 32 + 16, dt * 32, lane), db1, ak[dt]);
    }
    pipeline_reads<2 * (DTV + DTK), 2>();
  }

  // waves 4..7 hand their partial sums to waves 0..3 through LDS
  wait_all_loads();
  barrier();
  float* red = reinterpret_cast<float*>(smem) + cg * (DTK + DTV) * 16 * 64;
  if (half == 1) {
#pragma unroll
    for (int dt = 0; dt < DTK; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(red + ((dt * 4 + g4) * 64 + lane) * 4) =
            f32x4{ak[dt][g4 * 4], ak[dt][g4 * 4 + 1], ak[dt][g4 * 4 + 2], ak[dt][g4 * 4 + 3]};
#pragma unroll
    for (int dt = 0; dt < DTV; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(red + (((DTK + dt) * 4 + g4) * 64 + lane) * 4) =
            f32x4{av[dt][g4 * 4], av[dt][g4 * 4 + 1], av[dt][g4 * 4 + 2], av[dt][g4 * 4 + 3]};
  }
  barrier();
  if (half == 0 && key < p.Tk) {
    bf16_t* dkp = reinterpret_cast<bf16_t*>(p.dk) + b * p.dk_sb + kvh * p.dk_sh + (int64_t)key * p.dk_st;
    bf16_t* dvp = reinterpret_cast<bf16_t*>(p.dv) + b * p.dv_sb + kvh * p.dv_sh + (int64_t)key * p.dv_st;
#pragma unroll
    for (int dt = 0; dt < DTK; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(red + ((dt * 4 + g4) * 64 + lane) * 4);
        const int d = dt * 32 + g4 * 8 + lh * 4;
        *reinterpret_cast<u32x2*>(dkp + d) =
            u32x2{pack2((ak[dt][g4 * 4] + o[0]) * p.scale, (ak[dt][g4 * 4 + 1] + o[1]) * p.scale),
                  pack2((ak[dt][g4 * 4 + 2] + o[2]) * p.scale, (ak[dt][g4 * 4 + 3] + o[3]) * p.scale)};
      }
#pragma unroll
    for (int dt = 0; dt < DTV; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(red + (((DTK + dt) * 4 + g4) * 64 + lane) * 4);
        const int d = dt * 32 + g4 * 8 + lh * 4;
        *reinterpret_cast<u32x2*>(dvp + d) = u32x2{pack2(av[dt][g4 * 4] + o[0], av[dt][g4 * 4 + 1] + o[1]),
                                                   pack2(av[dt][g4 * 4 + 2] + o[2], av[dt][g4 * 4 + 3] + o[3])};
      }
  }
}

// ---------------------------------------------------------------------------
// 4. dQ: one workgroup per 32*NW folded query rows of one (b, kv head)
// ---------------------------------------------------------------------------
template <int DQK, int DV, int NW, int BN, bool DROP>
__global__ void __launch_bounds__(NW * 64) bwd_dq_kernel(const BwdParams p) {
  constexpr int BM = 32 * NW;
  constexpr int CPK = DQK / 8, CPV = DV / 8;
  constexpr int KS = DQK / 16, VS = DV / 16, DT = DQK / 32, MT = BN / 32, PKS = BN / 16;
  constexpr int KT_BYTES = BN * DQK * 2, STAGE = KT_BYTES + BN * DV * 2;
  // two stages: [K tile | V tile]
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, lh = lane >> 5;
  const int n_groups = p.B * p.Hkv;
  const int grp = blockIdx.x % n_groups, b = grp / p.Hkv, kvh = grp % p.Hkv;
  const int rows = p.g * p.Tq;  // folded rows of the group
  const int n_rt = (rows + BM - 1) / BM;
  const int tb = n_rt - 1 - (int)(blockIdx.x / n_groups);  // longest causal tiles first, every group
  const int f0 = tb * BM;
  const int f = f0 + wave * 32 + lq;
  const bool valid = f < rows;
  const int fc = valid ? f : rows - 1;
  const int h = kvh * p.g + fc / p.Tq, t = fc % p.Tq;
  const int off = p.Tk - p.Tq;
  const int up = p.causal ? 0 : p.win_right;  // keys after the diagonal a row may see (-1: unbounded)
  const int row_lim = !valid ? -1 : (up >= 0 ? min(t + off + up, p.Tk - 1) : p.Tk - 1);
  const int row_lo = p.win_left >= 0 ? t + off - p.win_left : 0;
  const int64_t lrow = ((int64_t)b * p.H + h) * p.Tq + t;
  const float lse = p.lse[lrow];
  const float l2 = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
  const float Dr = p.D[lrow];

  bf16x8 qf[KS], dof[VS];
  {
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)t * p.q_st;
    const bf16_t* dp = reinterpret_cast<const bf16_t*>(p.dout) + b * p.do_sb + h * p.do_sh + (int64_t)t * p.do_st;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + s * 16 + lh * 8);
#pragma unroll
    for (int s = 0; s < VS; ++s) dof[s] = *reinterpret_cast<const bf16x8*>(dp + s * 16 + lh * 8);
  }

  // keys this tile can see ([kstart, kend)), and keys every row of it sees
  // ([klfull, kfull)): blocks inside the latter need no per-score mask
  int kend = p.Tk, kfull = (f0 + BM <= rows) ? p.Tk : 0, kstart = 0, klfull = 0;
  {
    const int f_last = min(f0 + BM, rows) - 1;
    const bool one_head = f_last / p.Tq == f0 / p.Tq;
    const int t_hi = one_head ? f_last % p.Tq : p.Tq - 1;
    const int t_lo = one_head ? f0 % p.Tq : 0;
    if (up >= 0) {
      kend = max(0, min(p.Tk, t_hi + off + up + 1));
      kfull = min(kfull, max(0, t_lo + off + up + 1));
    }
    if (p.win_left >= 0) {
      kstart = min(p.Tk, max(0, t_lo + off - p.win_left));
      klfull = max(0, t_hi + off - p.win_left);
    }
  }
  const int nb = (kend + BN - 1) / BN, jb0 = kstart / BN;

  const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + b * p.k_sb + kvh * p.k_sh;
  const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + b * p.v_sb + kvh * p.v_sh;
  const uint32_t smem_s = lds_u32(smem);
  auto issue = [&](int j) {
    const uint32_t st = smem_s + (uint32_t)((j & 1) * STAGE);
    // with two waves per SIMD only the second wave of each SIMD issues the
    // tile loads, so the first keeps its MFMAs going while they queue
    // (measured: 4-5% on the 128-wide kernel)
    constexpr int NWI = NW >= 8 ? NW / 2 : NW;
    if (wave >= NW - NWI) {
      dma_tile<CPK, BN, NWI>(kbase, p.k_st, j * BN, p.Tk - 1, st, wave - (NW - NWI), lane);
      dma_tile<CPV, BN, NWI>(vbase, p.v_st, j * BN, p.Tk - 1, st + KT_BYTES, wave - (NW - NWI), lane);
    }
  };

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  // dropout: this row's keep words of block j (MT words), loaded one block
  // ahead so that their wait falls where the block's tiles are waited for
  const uint32_t* mrow = DROP ? p.keep + b * p.m_sb + h * p.m_sh + (int64_t)t * p.m_st : nullptr;
  // (the words of block j+1 are loaded into mw once block j's have been used,
  // so that no second set of registers holds them)
  uint32_t mw[MT];
  auto load_mask = [&](int j, uint32_t* dst) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) dst[mt] = (j * MT + mt < p.nwords) ? mrow[j * MT + mt] : 0u;
  };
  if constexpr (DROP) {
    if (nb > jb0) load_mask(jb0, mw);
  }

  if (nb > jb0) issue(jb0);
  for (int j = jb0; j < nb; ++j) {
    wait_all_loads();
    barrier();
    if (j + 1 < nb) issue(j + 1);
    const bf16_t* kt = reinterpret_cast<const bf16_t*>(smem + (j & 1) * STAGE);
    const bf16_t* vt = reinterpret_cast<const bf16_t*>(smem + (j & 1) * STAGE + KT_BYTES);
    f32x16 S[MT], dP[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        S[mt][i] = 0.f;
        dP[mt][i] = 0.f;
      }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int s = 0; s < (KS > VS ? KS : VS); ++s) {
        if (s < KS) S[mt] = mfma32(row_frag<CPK>(kt, mt * 32 + lq, s, lh), qf[s], S[mt]);
        if (s < VS) dP[mt] = mfma32(row_frag<CPV>(vt, mt * 32 + lq, s, lh), dof[s], dP[mt]);
      }
    }
    pipeline_reads<MT * (KS + VS), 1>();
    // S^T element i of tile mt is key j*BN + mt*32 + lh*4 + 8*(i/4) + i%4 of this lane's row
    float dS[MT * 16];
    const bool full = (j + 1) * BN <= kfull && j * BN >= klfull;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pr = __builtin_amdgcn_exp2f(fmaf(S[mt][i], p.c, -l2));
        if (!full) {
          const int kk = j * BN + mt * 32 + lh * 4 + 8 * (i >> 2) + (i & 3);
          pr = (kk <= row_lim && kk >= row_lo) ? pr : 0.f;
        }
        if constexpr (DROP) {
          const float z = ((mw[mt] >> (lh * 4 + 8 * (i >> 2) + (i & 3))) & 1u) ? p.inv_keep : 0.f;
          dS[mt * 16 + i] = pr * (z * dP[mt][i] - Dr);
        } else {
          dS[mt * 16 + i] = pr * (dP[mt][i] - Dr);
        }
      }
    if constexpr (DROP) {
      if (j + 1 < nb) load_mask(j + 1, mw);
    }
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) {
      const bf16x8 db = pack8(dS + ks * 8);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(tr_frag<CPK>(kt, ks * 16, dt * 32, lane), db, acc[dt]);
    }
    pipeline_reads<PKS * DT, 2>();
  }

  if (valid) {
    bf16_t* qo = reinterpret_cast<bf16_t*>(p.dq) + b * p.dq_sb + h * p.dq_sh + (int64_t)t * p.dq_st;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + lh * 4;
        *reinterpret_cast<u32x2*>(qo + d) = u32x2{pack2(acc[dt][g4 * 4] * p.scale, acc[dt][g4 * 4 + 1] * p.scale),
                                                  pack2(acc[dt][g4 * 4 + 2] * p.scale, acc[dt][g4 * 4 + 3] * p.scale)};
      }
  }
}

// ---------------------------------------------------------------------------
// 4b. dK/dV and dQ for 256- and 512-wide heads (d_qk = d_v = D). One wave
//     cannot hold a D-wide accumulator next to its operands, so the columns
//     are split into DS = D/128 slices of 128.
//     dK/dV: a workgroup owns 32*NG keys in NG groups of 32; a group has 2*DS
//     waves. K wave cs owns dK columns 128cs.. of the group's keys and forms
//     the partial S = Q K^T over those columns; V wave cs owns the same dV
//     columns and forms the partial dP = dO V^T. The partials go to LDS; each
//     wave of the group then owns 16/(2*DS) of the 16 accumulator elements of
//     every lane: it adds the partials of those elements in a fixed order,
//     forms P and dS, and writes them as bf16 over the partials it consumed;
//     after a barrier every wave reads the B operand it multiplies by (P for
//     dV, dS for dK). Three workgroup barriers per 32-row step, two waves per
//     SIMD; the Q and dO tiles are double-buffered through LDS.
//     dQ: 8 waves, groups of DS; wave (group gi, slice cs) owns columns
//     128cs.. of the group's 32 folded rows and forms partial S and dP over
//     them. The same reduce-scatter: wave cs adds the partials of 16/DS of
//     the elements in slice order, forms dS and writes it as bf16 over slice
//     0's partial of those elements; after a barrier every wave reads the
//     whole dS of its rows for dQ^T += K^T dS^T.
// ---------------------------------------------------------------------------
template <int D, int NG, bool DROP>
__global__ void __launch_bounds__(NG * 2 * (D / 128) * 64) bwd_dkdv_wide_kernel(const BwdParams p) {
  constexpr int DS = D / 128, GW = 2 * DS, NW = NG * GW, DC = 128;
  constexpr int EP = 16 / GW;  // accumulator elements of every lane a wave reduces
  constexpr int BNK = 32 * NG, BQ = 32;
  constexpr int CP = D / 8, KSC = DC / 16, DTC = DC / 32;
  constexpr int QT_BYTES = BQ * D * 2, STAGE = 2 * QT_BYTES;  // [Q tile | dO tile]
  constexpr int XW_BYTES = 4 * 64 * 16;                       // one wave's partial: [q][lane][4 floats]
  static_assert(EP == 2 || EP == 4, "two or four elements per wave");
  static_assert(2 * STAGE + NW * XW_BYTES <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE + NW * XW_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, lh = lane >> 5;
  const int gi = wave / GW, gw = wave % GW;
  const int role = gw / DS, cs = gw % DS;  // role 0: S and dK, role 1: dP and dV
  const int n_groups = p.B * p.Hkv;
  const int grp = blockIdx.x % n_groups, b = grp / p.Hkv, kvh = grp % p.Hkv;
  const int rsp = blockIdx.x / n_groups, sp = rsp % p.n_split;
  const int kb0 = (rsp / p.n_split) * BNK;  // the longest causal key blocks first
  const int h_lo = sp * p.g / p.n_split, h_hi = (sp + 1) * p.g / p.n_split;
  const int key = kb0 + gi * 32 + lq;
  const int keyc = min(key, p.Tk - 1);
  unsigned char* const xg = smem + 2 * STAGE + gi * GW * XW_BYTES;  // the group's partials
  auto xat = [&](int w, int q) { return xg + w * XW_BYTES + (q * 64 + lane) * 16; };

  // K (role 0) or V (role 1) of this lane's key over the wave's columns: the B
  // operand of the partial product
  bf16x8 kvf[KSC];
  {
    const bf16_t* src =
        role ? reinterpret_cast<const bf16_t*>(p.v) + b * p.v_sb + kvh * p.v_sh + (int64_t)keyc * p.v_st
             : reinterpret_cast<const bf16_t*>(p.k) + b * p.k_sb + kvh * p.k_sh + (int64_t)keyc * p.k_st;
    src += cs * DC;
#pragma unroll
    for (int s = 0; s < KSC; ++s) kvf[s] = *reinterpret_cast<const bf16x8*>(src + s * 16 + lh * 8);
  }
  f32x16 acc[DTC];
#pragma unroll
  for (int dt = 0; dt < DTC; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  const int off = p.Tk - p.Tq;
  const int up = p.causal ? 0 : p.win_right;
  const int t_first = up >= 0 ? max(0, kb0 - off - up) : 0;
  const int t_last = p.win_left >= 0 ? min(p.Tq - 1, kb0 + BNK - 1 - off + p.win_left) : p.Tq - 1;
  const int ntb = (p.Tq + BQ - 1) / BQ;
  const int tb0 = min(t_first / BQ, ntb);
  const int per_head = t_last < t_first ? 0 : max(0, min(ntb, t_last / BQ + 1) - tb0);
  const int n_it = (h_hi - h_lo) * per_head;
  const uint32_t smem_s = lds_u32(smem);

  auto issue = [&](int it) {
    const int hl = h_lo + it / per_head, t0 = (tb0 + it % per_head) * BQ;
    const int h = kvh * p.g + hl;
    const uint32_t st = smem_s + (uint32_t)((it & 1) * STAGE);
    dma_tile<CP, BQ, NW>(reinterpret_cast<const bf16_t*>(p.q) + b * p.q_sb + h * p.q_sh, p.q_st, t0, p.Tq - 1, st,
                         wave, lane);
    dma_tile<CP, BQ, NW>(reinterpret_cast<const bf16_t*>(p.dout) + b * p.do_sb + h * p.do_sh, p.do_st, t0, p.Tq - 1,
                         st + QT_BYTES, wave, lane);
  };
  // lse and D of the rows of this wave's elements (element e of a lane is
  // query row lh*4 + 8*(e/4) + e%4 of the tile), clamped to the last row, and
  // with dropout the keep word of each such row that holds the group's 32
  // keys; loaded one step ahead, before the step's tile loads are issued
  float L[EP], Dv[EP];
  uint32_t Mw[EP];
  const int wkey = min((kb0 + gi * 32) / 32, max(p.nwords - 1, 0));
  auto load_rows = [&](int it) {
    const int hl = h_lo + it / per_head, t0 = (tb0 + it % per_head) * BQ;
    const int h = kvh * p.g + hl;
    const int64_t rb = ((int64_t)b * p.H + h) * p.Tq;
#pragma unroll
    for (int k = 0; k < EP; ++k) {
      const int e = gw * EP + k;
      const int t = min(t0 + lh * 4 + 8 * (e >> 2) + (e & 3), p.Tq - 1);
      L[k] = p.lse[rb + t];
      Dv[k] = p.D[rb + t];
      if constexpr (DROP) Mw[k] = p.keep[b * p.m_sb + h * p.m_sh + (int64_t)t * p.m_st + wkey];
    }
  };

  if (n_it > 0) {
    load_rows(0);
    issue(0);
  }
  for (int it = 0; it < n_it; ++it) {
    wait_all_loads();
    barrier();  // tile it has landed everywhere; nobody reads the other stage or the partials any more
    float Lc[EP], Dc[EP];
    uint32_t Mc[EP];
#pragma unroll
    for (int k = 0; k < EP; ++k) {
      Lc[k] = L[k];
      Dc[k] = Dv[k];
      if constexpr (DROP) Mc[k] = Mw[k];
    }
    if (it + 1 < n_it) {
      load_rows(it + 1);
      issue(it + 1);
    }
    const int t0 = (tb0 + it % per_head) * BQ;
    const bf16_t* tl = reinterpret_cast<const bf16_t*>(smem + (it & 1) * STAGE + role * QT_BYTES);
    // the partial S (role 0) or dP (role 1) over the wave's columns
    f32x16 X;
#pragma unroll
    for (int i = 0; i < 16; ++i) X[i] = 0.f;
#pragma unroll
    for (int s = 0; s < KSC; ++s) X = mfma32(row_frag<CP>(tl, lq, cs * KSC + s, lh), kvf[s], X);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4*>(xat(gw, q)) = f32x4{X[4 * q], X[4 * q + 1], X[4 * q + 2], X[4 * q + 3]};
    barrier();
    // this wave's elements: the partials added in wave order, then P and dS
    float sv[EP], dv[EP];
#pragma unroll
    for (int k = 0; k < EP; ++k) sv[k] = dv[k] = 0.f;
#pragma unroll
    for (int c = 0; c < GW; ++c) {
      float v[EP];
      if constexpr (EP == 2) {
        const f32x2 x = *reinterpret_cast<const f32x2*>(xat(c, gw >> 1) + (gw & 1) * 8);
        v[0] = x[0];
        v[1] = x[1];
      } else {
        const f32x4 x = *reinterpret_cast<const f32x4*>(xat(c, gw));
        v[0] = x[0];
        v[1] = x[1];
        v[2] = x[2];
        v[3] = x[3];
      }
#pragma unroll
      for (int k = 0; k < EP; ++k) {
        if (c < DS)
          sv[k] += v[k];
        else
          dv[k] += v[k];
      }
    }
    float P[EP], dS[EP];
#pragma unroll
    for (int k = 0; k < EP; ++k) {
      const int e = gw * EP + k;
      const int t = t0 + lh * 4 + 8 * (e >> 2) + (e & 3);
      const int lim = t >= p.Tq ? -1 : (up >= 0 ? t + off + up : p.Tk - 1);
      const int lo = p.win_left >= 0 ? t + off - p.win_left : 0;
      float pr = __builtin_amdgcn_exp2f(fmaf(sv[k], p.c, -Lc[k] * kLog2e));
      pr = (key <= lim && key >= lo) ? pr : 0.f;
      if constexpr (DROP) {
        // dV takes the dropped probabilities; dS = P (Z dP - D)
        const float z = ((Mc[k] >> lq) & 1u) ? p.inv_keep : 0.f;
        P[k] = pr * z;
        dS[k] = pr * (z * dv[k] - Dc[k]);
      } else {
        P[k] = pr;
        dS[k] = pr * (dv[k] - Dc[k]);
      }
    }
    // written over wave 0's partial of these elements, which only this wave read
    if constexpr (EP == 2) {
      *reinterpret_cast<u32x2*>(xat(0, gw >> 1) + (gw & 1) * 8) = u32x2{pack2(P[0], P[1]), pack2(dS[0], dS[1])};
    } else {
      *reinterpret_cast<u32x4*>(xat(0, gw)) =
          u32x4{pack2(P[0], P[1]), pack2(P[2], P[3]), pack2(dS[0], dS[1]), pack2(dS[2], dS[3])};
    }
    barrier();
    // B operand: P for dV, dS for dK, elements 0..15 of this lane as bf16
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 c4 = *reinterpret_cast<const u32x4*>(xat(0, q));
      if constexpr (EP == 2) {  // {P 4q,4q+1 | dS 4q,4q+1 | P 4q+2,4q+3 | dS 4q+2,4q+3}
        w[2 * q] = role ? c4[0] : c4[1];
        w[2 * q + 1] = role ? c4[2] : c4[3];
      } else {  // {P 4q,4q+1 | P 4q+2,4q+3 | dS 4q,4q+1 | dS 4q+2,4q+3}
        w[2 * q] = role ? c4[0] : c4[2];
        w[2 * q + 1] = role ? c4[1] : c4[3];
      }
    }
    const bf16x8 b0 = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
    const bf16x8 b1 = __builtin_bit_cast(bf16x8, u32x4{w[4], w[5], w[6], w[7]});
#pragma unroll
    for (int dt = 0; dt < DTC; ++dt) {
      acc[dt] = mfma32(tr_frag<CP>(tl, 0, cs * DC + dt * 32, lane), b0, acc[dt]);
      acc[dt] = mfma32(tr_frag<CP>(tl, 16, cs * DC + dt * 32, lane), b1, acc[dt]);
    }
  }

  // dK^T (role 0, scaled) or dV^T (role 1) tile: lane holds key `key`, columns
  // 128 cs + dt*32 + 8*g4 + 4*lh .. +3
  if (key < p.Tk && p.n_split > 1) {
    float* pp = p.part + ((int64_t)(sp * n_groups + grp) * p.Tk + key) * (2 * D) + role * D + cs * DC;
#pragma unroll
    for (int dt = 0; dt < DTC; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + lh * 4;
        *reinterpret_cast<f32x4*>(pp + d) =
            f32x4{acc[dt][g4 * 4], acc[dt][g4 * 4 + 1], acc[dt][g4 * 4 + 2], acc[dt][g4 * 4 + 3]};
      }
  } else if (key < p.Tk) {
    bf16_t* dst =
        role ? reinterpret_cast<bf16_t*>(p.dv) + b * p.dv_sb + kvh * p.dv_sh + (int64_t)key * p.dv_st
             : reinterpret_cast<bf16_t*>(p.dk) + b * p.dk_sb + kvh * p.dk_sh + (int64_t)key * p.dk_st;
    dst += cs * DC;
    const float m = role ? 1.f : p.scale;
#pragma unroll
    for (int dt = 0; dt < DTC; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + lh * 4;
        *reinterpret_cast<u32x2*>(dst + d) = u32x2{pack2(acc[dt][g4 * 4] * m, acc[dt][g4 * 4 + 1] * m),
                                                   pack2(acc[dt][g4 * 4 + 2] * m, acc[dt][g4 * 4 + 3] * m)};
      }
  }
}

template <int D, int NG, bool DROP>
__global__ void __launch_bounds__(NG * (D / 128) * 64) bwd_dq_wide_kernel(const BwdParams p) {
  constexpr int DS = D / 128, NW = NG * DS, DC = 128;
  constexpr int BM = 32 * NG, BN = 32;
  constexpr int CP = D / 8, KSC = DC / 16, DTC = DC / 32;
  constexpr int KT_BYTES = BN * D * 2;
  constexpr int XS_FLOATS = NW * 2 * 16 * 64;
  // K tiles are double-buffered; V tiles too where LDS allows, else one V
  // stage is refilled as soon as every wave has taken its dP from it
  constexpr int NVS = 4 * KT_BYTES + XS_FLOATS * 4 <= 160 * 1024 ? 2 : 1;
  constexpr int V_OFF = 2 * KT_BYTES, XS_OFF = V_OFF + NVS * KT_BYTES;
  static_assert(XS_OFF + XS_FLOATS * 4 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[XS_OFF + XS_FLOATS * 4];
  constexpr int EP = 16 / DS;                // accumulator elements of every lane a wave reduces
  constexpr int XW_BYTES = 2 * 4 * 64 * 16;  // one wave's partials: [S | dP][q][lane][4 floats]
  static_assert(NW * XW_BYTES == XS_FLOATS * 4, "partials area");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, lh = lane >> 5;
  const int gi = wave / DS, cs = wave % DS;
  const int n_groups = p.B * p.Hkv;
  const int grp = blockIdx.x % n_groups, b = grp / p.Hkv, kvh = grp % p.Hkv;
  unsigned char* const xg = smem + XS_OFF + gi * DS * XW_BYTES;  // the group's partials
  auto xat = [&](int w, int m, int q) { return xg + w * XW_BYTES + ((m * 4 + q) * 64 + lane) * 16; };
  const int rows = p.g * p.Tq;
  const int n_rt = (rows + BM - 1) / BM;
  const int tb = n_rt - 1 - (int)(blockIdx.x / n_groups);  // longest causal tiles first
  const int f0 = tb * BM;
  const int f = f0 + gi * 32 + lq;
  const bool valid = f < rows;
  const int fc = valid ? f : rows - 1;
  const int h = kvh * p.g + fc / p.Tq, t = fc % p.Tq;
  const int off = p.Tk - p.Tq;
  const int up = p.causal ? 0 : p.win_right;
  const int row_lim = !valid ? -1 : (up >= 0 ? min(t + off + up, p.Tk - 1) : p.Tk - 1);
  const int row_lo = p.win_left >= 0 ? t + off - p.win_left : 0;
  const int64_t lrow = ((int64_t)b * p.H + h) * p.Tq + t;
  const float lse = p.lse[lrow];
  const float l2 = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
  const float Dr = p.D[lrow];

  // q and dO of this lane's row over the wave's columns (B operands of S^T and dP^T)
  bf16x8 qf[KSC], dof[KSC];
  {
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)t * p.q_st + cs * DC;
    const bf16_t* dp =
        reinterpret_cast<const bf16_t*>(p.dout) + b * p.do_sb + h * p.do_sh + (int64_t)t * p.do_st + cs * DC;
#pragma unroll
    for (int s = 0; s < KSC; ++s) {
      qf[s] = *reinterpret_cast<const bf16x8*>(qp + s * 16 + lh * 8);
      dof[s] = *reinterpret_cast<const bf16x8*>(dp + s * 16 + lh * 8);
    }
  }

  // keys the workgroup's rows can see ([kstart, kend))
  int kend = p.Tk, kstart = 0;
  {
    const int f_last = min(f0 + BM, rows) - 1;
    const bool one_head = f_last / p.Tq == f0 / p.Tq;
    const int t_hi = one_head ? f_last % p.Tq : p.Tq - 1;
    const int t_lo = one_head ? f0 % p.Tq : 0;
    if (up >= 0) kend = max(0, min(p.Tk, t_hi + off + up + 1));
    if (p.win_left >= 0) kstart = min(p.Tk, max(0, t_lo + off - p.win_left));
  }
  const int nb = (kend + BN - 1) / BN, jb0 = kstart / BN;

  const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + b * p.k_sb + kvh * p.k_sh;
  const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + b * p.v_sb + kvh * p.v_sh;
  const uint32_t smem_s = lds_u32(smem);
  auto issue_k = [&](int j) {
    dma_tile<CP, BN, NW>(kbase, p.k_st, j * BN, p.Tk - 1, smem_s + (uint32_t)((j & 1) * KT_BYTES), wave, lane);
  };
  auto issue_v = [&](int j) {
    dma_tile<CP, BN, NW>(vbase, p.v_st, j * BN, p.Tk - 1,
                         smem_s + (uint32_t)(V_OFF + (NVS == 2 ? (j & 1) : 0) * KT_BYTES), wave, lane);
  };

  f32x16 acc[DTC];
#pragma unroll
  for (int dt = 0; dt < DTC; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  // dropout: the keep word of this lane's row for key block j (32 keys),
  // loaded a block ahead so that its wait falls where the block's tiles are
  // waited for
  const uint32_t* mrow = DROP ? p.keep + b * p.m_sb + h * p.m_sh + (int64_t)t * p.m_st : nullptr;
  uint32_t mw = 0u;
  if constexpr (DROP) {
    if (nb > jb0) mw = jb0 < p.nwords ? mrow[jb0] : 0u;
  }
  if (nb > jb0) {
    issue_k(jb0);
    issue_v(jb0);
  }
  for (int j = jb0; j < nb; ++j) {
    wait_all_loads();
    barrier();  // tile j has landed everywhere; nobody reads the stages it+1 refills any more
    if (j + 1 < nb) {
      issue_k(j + 1);
      if constexpr (NVS == 2) issue_v(j + 1);
    }
    const bf16_t* kt = reinterpret_cast<const bf16_t*>(smem + (j & 1) * KT_BYTES);
    const bf16_t* vt = reinterpret_cast<const bf16_t*>(smem + V_OFF + (NVS == 2 ? (j & 1) : 0) * KT_BYTES);
    // partial S^T and dP^T over the wave's columns; element i is key
    // j*BN + lh*4 + 8*(i/4) + i%4 of this lane's row
    f32x16 S, dP;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      S[i] = 0.f;
      dP[i] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < KSC; ++s) {
      S = mfma32(row_frag<CP>(kt, lq, cs * KSC + s, lh), qf[s], S);
      dP = mfma32(row_frag<CP>(vt, lq, cs * KSC + s, lh), dof[s], dP);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<f32x4*>(xat(cs, 0, q)) = f32x4{S[4 * q], S[4 * q + 1], S[4 * q + 2], S[4 * q + 3]};
      *reinterpret_cast<f32x4*>(xat(cs, 1, q)) = f32x4{dP[4 * q], dP[4 * q + 1], dP[4 * q + 2], dP[4 * q + 3]};
    }
    barrier();
    if constexpr (NVS == 1)  // every wave has its dP partial: the V stage is free
      if (j + 1 < nb) issue_v(j + 1);
    // this wave's elements (keys) of the lane's row: the partials added in
    // slice order, then dS, written as bf16 over slice 0's S partial of
    // those elements (read by this wave only)
    float sv[EP], dv[EP];
#pragma unroll
    for (int k = 0; k < EP; ++k) sv[k] = dv[k] = 0.f;
#pragma unroll
    for (int c = 0; c < DS; ++c)
#pragma unroll
      for (int q4 = 0; q4 < EP / 4; ++q4) {
        const f32x4 xsv = *reinterpret_cast<const f32x4*>(xat(c, 0, cs * (EP / 4) + q4));
        const f32x4 xdv = *reinterpret_cast<const f32x4*>(xat(c, 1, cs * (EP / 4) + q4));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          sv[q4 * 4 + k] += xsv[k];
          dv[q4 * 4 + k] += xdv[k];
        }
      }
    uint32_t dw[EP / 2];
#pragma unroll
    for (int k = 0; k < EP; k += 2) {
      float d2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = cs * EP + k + u;
        const int kk = j * BN + lh * 4 + 8 * (e >> 2) + (e & 3);
        float pr = __builtin_amdgcn_exp2f(fmaf(sv[k + u], p.c, -l2));
        pr = (kk <= row_lim && kk >= row_lo) ? pr : 0.f;
        if constexpr (DROP) {
          const float z = ((mw >> (lh * 4 + 8 * (e >> 2) + (e & 3))) & 1u) ? p.inv_keep : 0.f;
          d2[u] = pr * (z * dv[k + u] - Dr);
        } else {
          d2[u] = pr * (dv[k + u] - Dr);
        }
      }
      dw[k / 2] = pack2(d2[0], d2[1]);
    }
    if constexpr (DROP) {
      if (j + 1 < nb) mw = j + 1 < p.nwords ? mrow[j + 1] : 0u;
    }
    if constexpr (EP == 4) {
      *reinterpret_cast<u32x2*>(xat(0, 0, cs)) = u32x2{dw[0], dw[1]};
    } else {
      *reinterpret_cast<u32x4*>(xat(0, 0, 2 * cs)) = u32x4{dw[0], dw[1], dw[2], dw[3]};
    }
    barrier();
    // dS of elements 0..15 of this lane as bf16 (the B operand)
    uint32_t w[8];
    if constexpr (EP == 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 c2 = *reinterpret_cast<const u32x2*>(xat(0, 0, q));
        w[2 * q] = c2[0];
        w[2 * q + 1] = c2[1];
      }
    } else {
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const u32x4 c4 = *reinterpret_cast<const u32x4*>(xat(0, 0, 2 * o));
        w[4 * o] = c4[0];
        w[4 * o + 1] = c4[1];
        w[4 * o + 2] = c4[2];
        w[4 * o + 3] = c4[3];
      }
    }
    const bf16x8 db0 = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
    const bf16x8 db1 = __builtin_bit_cast(bf16x8, u32x4{w[4], w[5], w[6], w[7]});
#pragma unroll
    for (int dt = 0; dt < DTC; ++dt) {
      acc[dt] = mfma32(tr_frag<CP>(kt, 0, cs * DC + dt * 32, lane), db0, acc[dt]);
      acc[dt] = mfma32(tr_frag<CP>(kt, 16, cs * DC + dt * 32, lane), db1, acc[dt]);
    }
  }

  if (valid) {
    bf16_t* qo = reinterpret_cast<bf16_t*>(p.dq) + b * p.dq_sb + h * p.dq_sh + (int64_t)t * p.dq_st + cs * DC;
#pragma unroll
    for (int dt = 0; dt < DTC; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + lh * 4;
        *reinterpret_cast<u32x2*>(qo + d) = u32x2{pack2(acc[dt][g4 * 4] * p.scale, acc[dt][g4 * 4 + 1] * p.scale),
                                                  pack2(acc[dt][g4 * 4 + 2] * p.scale, acc[dt][g4 * 4 + 3] * p.scale)};
      }
  }
}

// ---------------------------------------------------------------------------
// 7. Forward with attention dropout. The keep mask is an input that the
//    backward reads too, so the two cannot disagree on it (the
//    TransformerEngine page's review names a context-parallel backward that
//    lost the dropout probability and RNG state the forward used). The dQ
//    kernel's tiling: 32 folded query rows per wave with Q in registers, 64-key
//    K and V tiles through LDS, S^T = K Q^T, an online softmax per row (the
//    two lane halves hold different keys of a row), O^T += V^T (P keep)^T.
//    The denominator takes every visible probability; only the product with
//    V sees the mask, and the kept ones are scaled by 1 / (1 - p) at the end.
// ---------------------------------------------------------------------------
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold of the online softmax (log2 units)

template <int DQK, int DV>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DQK + DV > 320 ? 1 : 2)))
fwd_dropout_kernel(const BwdParams p) {
  constexpr int NW = 4, BN = 64, BM = 32 * NW;
  constexpr int CPK = DQK / 8, CPV = DV / 8;
  constexpr int KS = DQK / 16, DT = DV / 32, MT = BN / 32, PKS = BN / 16;
  constexpr int KT_BYTES = BN * DQK * 2, STAGE = KT_BYTES + BN * DV * 2;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, lh = lane >> 5;
  const int n_groups = p.B * p.Hkv;
  const int grp = blockIdx.x % n_groups, b = grp / p.Hkv, kvh = grp % p.Hkv;
  const int rows = p.g * p.Tq;  // folded rows of the group
  const int n_rt = (rows + BM - 1) / BM;
  const int tb = n_rt - 1 - (int)(blockIdx.x / n_groups);  // longest causal tiles first
  const int f0 = tb * BM;
  const int f = f0 + wave * 32 + lq;
  const bool valid = f < rows;
  const int fc = valid ? f : rows - 1;
  const int h = kvh * p.g + fc / p.Tq, t = fc % p.Tq;
  const int off = p.Tk - p.Tq;
  const int up = p.causal ? 0 : p.win_right;
  const int row_lim = !valid ? -1 : (up >= 0 ? min(t + off + up, p.Tk - 1) : p.Tk - 1);
  const int row_lo = p.win_left >= 0 ? t + off - p.win_left : 0;

  bf16x8 qf[KS];
  {
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)t * p.q_st;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + s * 16 + lh * 8);
  }
  int kend = p.Tk, kfull = (f0 + BM <= rows) ? p.Tk : 0, kstart = 0, klfull = 0;
  {
    const int f_last = min(f0 + BM, rows) - 1;
    const bool one_head = f_last / p.Tq == f0 / p.Tq;
    const int t_hi = one_head ? f_last % p.Tq : p.Tq - 1;
    const int t_lo = one_head ? f0 % p.Tq : 0;
    if (up >= 0) {
      kend = max(0, min(p.Tk, t_hi + off + up + 1));
      kfull = min(kfull, max(0, t_lo + off + up + 1));
    }
    if (p.win_left >= 0) {
      kstart = min(p.Tk, max(0, t_lo + off - p.win_left));
      klfull = max(0, t_hi + off - p.win_left);
    }
  }
  const int nb = (kend + BN - 1) / BN, jb0 = kstart / BN;

  const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + b * p.k_sb + kvh * p.k_sh;
  const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + b * p.v_sb + kvh * p.v_sh;
  const uint32_t smem_s = lds_u32(smem);
  auto issue = [&](int j) {
    const uint32_t st = smem_s + (uint32_t)((j & 1) * STAGE);
    dma_tile<CPK, BN, NW>(kbase, p.k_st, j * BN, p.Tk - 1, st, wave, lane);
    dma_tile<CPV, BN, NW>(vbase, p.v_st, j * BN, p.Tk - 1, st + KT_BYTES, wave, lane);
  };
  // this row's keep words of block j, loaded one block ahead
  const uint32_t* mrow = p.keep + b * p.m_sb + h * p.m_sh + (int64_t)t * p.m_st;
  uint32_t mw[MT], mwn[MT];
  auto load_mask = [&](int j, uint32_t* dst) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) dst[mt] = (j * MT + mt < p.nwords) ? mrow[j * MT + mt] : 0u;
  };

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  if (nb > jb0) {
    load_mask(jb0, mw);
    issue(jb0);
  }
  for (int j = jb0; j < nb; ++j) {
    wait_all_loads();
    barrier();
    if (j + 1 < nb) {
      issue(j + 1);
      load_mask(j + 1, mwn);
    }
    const bf16_t* kt = reinterpret_cast<const bf16_t*>(smem + (j & 1) * STAGE);
    const bf16_t* vt = reinterpret_cast<const bf16_t*>(smem + (j & 1) * STAGE + KT_BYTES);
    f32x16 S[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[mt][i] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int s = 0; s < KS; ++s) S[mt] = mfma32(row_frag<CPK>(kt, mt * 32 + lq, s, lh), qf[s], S[mt]);
    pipeline_reads<MT * KS, 1>();
    // S^T element i of tile mt is key j*BN + mt*32 + lh*4 + 8*(i/4) + i%4 of this lane's row
    const bool full = (j + 1) * BN <= kfull && j * BN >= klfull;
    // four partial maxima and sums keep the dependency chains short
    float mx4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (!full) {
          const int kk = j * BN + mt * 32 + lh * 4 + 8 * (i >> 2) + (i & 3);
          if (!(kk <= row_lim && kk >= row_lo)) S[mt][i] = -INFINITY;
        }
        mx4[i & 3] = fmaxf(mx4[i & 3], S[mt][i]);
      }
    float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));  // the other half of the row's keys
    // lazy rescale: the running maximum only moves when a score exceeds it by
    // more than kRescaleLog2 (log2 units), so the exp2 arguments stay below
    // that bound and the accumulator is rescaled on the first blocks only
    const float mnew = fmaxf(m_run, mx);
    const bool grow = (mnew - m_run) * p.c > kRescaleLog2;  // false when both are -inf
    if (__any(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - mnew) * p.c) : 1.f;
      if (grow) m_run = mnew;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * p.c;
    float pd[MT * 16];
    float rs4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(fmaf(S[mt][i], p.c, -mc));
        rs4[i & 3] += e;
        pd[mt * 16 + i] = ((mw[mt] >> (lh * 4 + 8 * (i >> 2) + (i & 3))) & 1u) ? e : 0.f;
      }
    l_run += (rs4[0] + rs4[1]) + (rs4[2] + rs4[3]);
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) {
      const bf16x8 pb = pack8(pd + ks * 8);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(tr_frag<CPV>(vt, ks * 16, dt * 32, lane), pb, acc[dt]);
    }
    pipeline_reads<PKS * DT, 2>();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) mw[mt] = mwn[mt];
  }

  // epilogue: the row's denominator (both halves, the sink), O and lse
  const float l = l_run + __shfl_xor(l_run, 32, 64);
  const float sk = p.sinks != nullptr ? p.sinks[h] : -INFINITY;
  float factor = 0.f, lse = sk;
  if (m_run != -INFINITY) {
    const float ms = m_run * p.scale;
    const float mtot = fmaxf(ms, sk);
    const float a = __builtin_amdgcn_exp2f((ms - mtot) * kLog2e);
    const float den = l * a + (sk != -INFINITY ? __builtin_amdgcn_exp2f((sk - mtot) * kLog2e) : 0.f);
    factor = a / den * p.inv_keep;
    lse = mtot + __builtin_amdgcn_logf(den) * kLn2;
  }
  if (valid) {
    bf16_t* op = reinterpret_cast<bf16_t*>(p.fwd_out) + b * p.o_sb + h * p.o_sh + (int64_t)t * p.o_st;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + lh * 4;
        *reinterpret_cast<u32x2*>(op + d) = u32x2{pack2(acc[dt][g4 * 4] * factor, acc[dt][g4 * 4 + 1] * factor),
                                                  pack2(acc[dt][g4 * 4 + 2] * factor, acc[dt][g4 * 4 + 3] * factor)};
      }
    if (lh == 0) p.fwd_lse[((int64_t)b * p.H + h) * p.Tq + t] = lse;
  }
}

// ---------------------------------------------------------------------------
// 8. Sparse top-k decode over an fp8 pool (the sparse fp8 decode the
//    TensorRT-LLM page names among FlashMLA's kernels): pool rows of 512 OCP
//    E4M3 codes with one fp32 scale per 128 columns, decoded in the kernel
//    (only the gathered rows are ever converted, never the pool). One
//    workgroup of 8 waves per (query, range of its slots); per step of 32
//    slots the rows' codes and scales arrive by DMA into one of four staging
//    buffers (three steps ahead, explicit vmcnt accounting). The MFMA operands
//    come straight from the staged codes: a lane converts the 8 codes of its
//    operand to bf16 (v_cvt_scalef32_pk_bf16_fp8 with scale 1: exact, an E4M3
//    value has 4 significant bits), row-wise for S^T and through the 8-bit
//    transposed LDS read (lane i of a 16-lane group gets byte i of 8
//    consecutive 16-byte rows) for X^T. Wave (hg, sq) forms S^T for heads
//    32 hg.. over columns 128 sq.., which is exactly one scale block, so it
//    multiplies its partial by each key's scale of that block in fp32; the
//    four partials are summed through LDS in a fixed order; the online softmax
//    is per head; O^T += X^T (P s)^T on the wave's 128 output columns, the
//    same block's scales applied to P before it is rounded for the product.
//    No decoded value is ever rounded. Each range writes its normalised O and
//    its lse without the sink; the split-KV merge adds the sink and combines
//    the ranges.
//
//    Staged row r keeps its 16-byte chunk c at position c ^ (r % 16) (the DMA
//    lanes fetch the chunks in that order), so the 32 rows a read touches
//    fall in distinct bank groups. S^T's MFMA row m reads staged row pi(m)
//    (bits 2 and 3 of m swapped): then the 8 scores a lane hands to each
//    X^T P^T product belong to 8 consecutive staged rows, the rows one
//    transposed read returns.
// ---------------------------------------------------------------------------
constexpr int kFp8Stages = 4, kFp8IdxCap = 4096;

// 8 E4M3 codes (two words) -> 8 bf16, exactly
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// staged row of S^T's MFMA row m: bits 2 and 3 swapped
__device__ __forceinline__ int fp8_row_of(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__global__ void __launch_bounds__(512) sparse_fp8_kernel(const SpFp8Params p) {
  constexpr int D = 512, BN = 32;
  constexpr int STG = BN * D;               // codes of one step
  constexpr int SCB = BN * 16;              // scales of one step (4 per row)
  constexpr int XB_BYTES = 8 * 16 * 64 * 4; // partial S^T exchange
  constexpr int NS = kFp8Stages, PD = NS - 1;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NS * STG + NS * SCB + XB_BYTES + kFp8IdxCap * 4];
  unsigned char* const stg = smem;
  float* const scl = reinterpret_cast<float*>(smem + NS * STG);
  float* const xb = reinterpret_cast<float*>(smem + NS * STG + NS * SCB);
  int32_t* const sidx = reinterpret_cast<int32_t*>(smem + NS * STG + NS * SCB + XB_BYTES);

  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, lh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 1, sq = wave >> 1;
  const int s = blockIdx.x, r = blockIdx.y;
  const int hd = hg * 32 + lq;
  const int k_lo = r * p.split_keys, k_hi = min(p.topk, k_lo + p.split_keys);
  const int nk = max(0, k_hi - k_lo);
  const int nblk = (nk + BN - 1) / BN;

  // the range's slots into LDS (-1: past the range, or outside the pool)
  const int32_t* ixrow = p.idx + (int64_t)s * p.idx_ss + k_lo;
  for (int e = tid; e < nblk * BN; e += 512) {
    const int ix = e < nk ? ixrow[e] : -1;
    sidx[e] = (ix >= 0 && ix < p.N) ? ix : -1;
  }
  // B operands of S^T: this lane's head, columns 128 sq + 16 k + 8 lh
  bf16x8 qf[8];
  {
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)s * p.q_ss + (int64_t)hd * p.q_sh + sq * 128 + lh * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) qf[k] = *reinterpret_cast<const bf16x8*>(qp + k * 16);
#pragma unroll
    for (int k = 0; k < 8; ++k) asm volatile("" ::"v"(qf[k]));  // wait for them here, not in the loop
  }
  __syncthreads();

  // step j: wave w gathers rows 4w .. 4w+3 (two rows of 512 codes per
  // instruction: lanes 0-31 the first, 32-63 the second; lane lq fetches
  // chunk lq ^ (row % 16)); wave 0 also the 32 rows' scales (16 bytes each,
  // lanes 0-31). Skipped slots read row 0.
  const uint32_t stg_s = lds_u32(stg), scl_s = lds_u32(scl);
  auto issue = [&](int j) {
    const uint32_t buf = (uint32_t)(j % NS);
    const int myix = sidx[j * BN + lq];
    const int myrow = myix < 0 ? 0 : myix;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int r0 = wave * 4 + 2 * m;
      const int ra = __builtin_amdgcn_readlane(myrow, r0), rb = __builtin_amdgcn_readlane(myrow, r0 + 1);
      const int rowl = lh ? rb : ra;
      const uint32_t chunk = (uint32_t)(lq ^ ((r0 + lh) & 15));
      dma16(p.codes, (uint32_t)rowl * (uint32_t)p.c_sn + 16u * chunk, stg_s + buf * STG + 512u * r0);
    }
    if (wave == 0 && lane < BN) dma16(p.scales, 4u * (uint32_t)myrow * (uint32_t)p.s_sn, scl_s + buf * SCB);
  };
  const int per_step = wave == 0 ? 3 : 2;  // this wave's loads of one step

  // this lane's staged row for S^T, and its rows / column chunk for X^T
  const int srow = fp8_row_of(lq);
  const int g16 = lane >> 4, j16 = lane & 15;
  const int trow = 8 * (g16 >> 1) + (j16 >> 1);  // + 16 ks

  f32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int j = 0; j < PD && j < nblk; ++j) issue(j);
  for (int j = 0; j < nblk; ++j) {
    // step j's loads have landed once at most the later steps' are in flight
    wait_vmcnt_dyn(per_step * min(PD - 1, nblk - 1 - j));
    barrier();
    if (j + PD < nblk) issue(j + PD);
    const unsigned char* st = stg + (j % NS) * STG;
    // partial S^T over columns 128 sq .. 128 sq + 127 (chunks 8 sq + k)
    f32x16 S;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = 0.f;
    {
      const unsigned char* rp = st + srow * D + 8 * lh;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(rp + (((8 * sq + k) ^ (srow & 15)) << 4));
        S = mfma32(fp8x8_to_bf16(w[0], w[1]), qf[k], S);
      }
    }
    // S^T element i: MFMA row lh*4 + 8*(i/4) + i%4, staged row 16*(i/8) + 8*lh + i%8
    float ks[16];
    {
      const float* sc = scl + (j % NS) * (SCB / 4) + sq;
#pragma unroll
      for (int i = 0; i < 16; ++i) ks[i] = sc[4 * (16 * (i >> 3) + 8 * lh + (i & 7))];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] *= ks[i];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<f32x4*>(xb + ((wave * 4 + g4) * 64 + lane) * 4) =
          f32x4{S[g4 * 4], S[g4 * 4 + 1], S[g4 * 4 + 2], S[g4 * 4 + 3]};
    barrier();
    // the four partials of these heads, summed in the same order by all four waves
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f32x4 t4 = *reinterpret_cast<const f32x4*>(xb + (((hg + 0) * 4 + g4) * 64 + lane) * 4);
#pragma unroll
      for (int o = 1; o < 4; ++o) t4 += *reinterpret_cast<const f32x4*>(xb + (((hg + 2 * o) * 4 + g4) * 64 + lane) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) S[g4 * 4 + e] = t4[e];
    }
    const uint32_t skip = (uint32_t)__ballot(sidx[j * BN + lq] < 0);
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((skip >> (16 * (i >> 3) + 8 * lh + (i & 7))) & 1u) S[i] = -INFINITY;
      mx = fmaxf(mx, S[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m_run, mx);
    const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f((m_run - mnew) * p.c);
    m_run = mnew;
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] *= alpha;
    const float mc = (mnew == -INFINITY) ? 0.f : mnew * p.c;
    float pr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(fmaf(S[i], p.c, -mc));
      l_run += e;
      pr[i] = e * ks[i];  // the values of these columns are code * scale
    }
    // X^T for output columns 128 sq + 32 t + (lane % 32), staged rows 16 ks + 8 lh + 0..7
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pb = pack8(pr + kk * 8);
      const int row = 16 * kk + trow;
      const unsigned char* rp = st + row * D + 8 * (j16 & 1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int chunk = 8 * sq + 2 * t + (g16 & 1);
        const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2*)(rp + ((chunk ^ (row & 15)) << 4)));
        acc[t] = mfma32(fp8x8_to_bf16((uint32_t)w[0], (uint32_t)w[1]), pb, acc[t]);
      }
    }
  }

  // this range's partial: O normalised by its own denominator, lse without the sink
  const float l = l_run + __shfl_xor(l_run, 32, 64);
  const bool any = m_run != -INFINITY && l > 0.f;
  const float inv = any ? 1.f / l : 0.f;
  const int64_t R = (int64_t)p.Sq * p.Hq, orow = (int64_t)r * R + (int64_t)s * p.Hq + hd;
  float* const po = p.part_o + orow * D;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int col = sq * 128 + t * 32 + g4 * 8 + lh * 4;
      *reinterpret_cast<f32x4*>(po + col) = f32x4{acc[t][g4 * 4] * inv, acc[t][g4 * 4 + 1] * inv,
                                                  acc[t][g4 * 4 + 2] * inv, acc[t][g4 * 4 + 3] * inv};
    }
  if (sq == 0 && lh == 0) p.part_lse[orow] = any ? m_run * p.scale + __builtin_amdgcn_logf(l) * kLn2 : -INFINITY;
}

// dK and dV from the head-split partials: four columns a thread, the splits
// added in order (so the result does not depend on the launch's timing)
template <int D>
__global__ void __launch_bounds__(256) bwd_wide_reduce_kernel(const BwdParams p) {
  constexpr int C4 = 2 * D / 4;  // four-column units of one key's [dK | dV] row
  const int64_t n_keys = (int64_t)p.B * p.Hkv * p.Tk;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= n_keys * C4) return;
  const int64_t row = u / C4;
  const int c = (int)(u % C4) * 4;
  const int grp = (int)(row / p.Tk), key = (int)(row % p.Tk), b = grp / p.Hkv, kvh = grp % p.Hkv;
  const int64_t split_stride = n_keys * 2 * D;
  const float* src = p.part + row * 2 * D + c;
  f32x4 a = *reinterpret_cast<const f32x4*>(src);
  for (int s = 1; s < p.n_split; ++s) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(src + s * split_stride);
    a[0] += x[0];
    a[1] += x[1];
    a[2] += x[2];
    a[3] += x[3];
  }
  bf16_t* dst;
  float m = 1.f;
  if (c < D) {
    dst = reinterpret_cast<bf16_t*>(p.dk) + b * p.dk_sb + kvh * p.dk_sh + (int64_t)key * p.dk_st + c;
    m = p.scale;
  } else {
    dst = reinterpret_cast<bf16_t*>(p.dv) + b * p.dv_sb + kvh * p.dv_sh + (int64_t)key * p.dv_st + (c - D);
  }
  *reinterpret_cast<u32x2*>(dst) = u32x2{pack2(a[0] * m, a[1] * m), pack2(a[2] * m, a[3] * m)};
}

// 256- and 512-wide heads: column-split dK/dV and dQ kernels (8 waves a workgroup each)
template <int D, bool DROP>
int launch_bwd_wide(const BwdParams& p, void* stream) {
  constexpr int NG = 512 / D, NW = NG * 2 * (D / 128);          // dK/dV: 8 waves
  constexpr int NGQ = 1024 / D, NWQ = NGQ * (D / 128);        // dQ: 8 waves
  if (p.n_split < 1 || p.n_split > p.g || (p.n_split > 1 && p.part == nullptr)) return (int)hipErrorInvalidValue;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t R = (int64_t)p.B * p.H * p.Tq;
  if (R > 0) {
    constexpr int RPB = 4 * (64 / (D / 8));  // rows per block of the dot kernel
    hipLaunchKernelGGL(bwd_dot_kernel<D>, dim3((unsigned)((R + RPB - 1) / RPB)), dim3(256), 0, st, p);
    if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
  }
  if (p.sinks != nullptr && p.dsinks != nullptr) {
    hipLaunchKernelGGL(bwd_dsink_kernel, dim3(p.H), dim3(256), 0, st, p);
    if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
  }
  if (p.Tk > 0) {
    const int nkb = (p.Tk + 32 * NG - 1) / (32 * NG);
    hipLaunchKernelGGL((bwd_dkdv_wide_kernel<D, NG, DROP>), dim3(nkb * p.n_split * p.B * p.Hkv), dim3(NW * 64), 0,
                       st, p);
    if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
    if (p.n_split > 1) {
      const int64_t units = (int64_t)p.B * p.Hkv * p.Tk * (2 * D / 4);
      hipLaunchKernelGGL(bwd_wide_reduce_kernel<D>, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st, p);
      if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
    }
  }
  if (p.Tq > 0) {
    const int rows = p.g * p.Tq;
    const int nrt = (rows + 32 * NGQ - 1) / (32 * NGQ);
    hipLaunchKernelGGL((bwd_dq_wide_kernel<D, NGQ, DROP>), dim3(nrt * p.B * p.Hkv), dim3(NWQ * 64), 0, st, p);
    if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
  }
  return 0;
}

template <int DQK, int DV, bool DROP>
int launch_bwd_cfg(const BwdParams& p, void* stream) {
  // dQ: two waves per SIMD where the registers allow it (d_qk + d_v <= 256)
  // (the dQ kernel with dropout and 128-wide heads takes 32-key blocks: with 64
  // its mask words put it one register over the two-wave budget); the
  // one-wave d192 kernels take 128-key (dQ) and 64-row (dK/dV) steps, which
  // their register room allows (measured 3% and 9% faster than 64 and 32;
  // with dropout's mask words the d192 dQ keeps 64-key blocks, 128 spill)
  constexpr int NW_KV = 4, NW_Q = DQK + DV > 256 ? 4 : 8;
  constexpr int BN_Q = (DROP && DQK + DV == 256) ? 32 : (DQK + DV > 256 && !DROP ? 128 : 64);
  constexpr int BQ_KV = 64;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t R = (int64_t)p.B * p.H * p.Tq;
  if (R > 0) {
    constexpr int RPB = 4 * (64 / (DV / 8));  // rows per block of the dot kernel
    hipLaunchKernelGGL(bwd_dot_kernel<DV>, dim3((unsigned)((R + RPB - 1) / RPB)), dim3(256), 0, st, p);
    if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
  }
  if (p.sinks != nullptr && p.dsinks != nullptr) {
    hipLaunchKernelGGL(bwd_dsink_kernel, dim3(p.H), dim3(256), 0, st, p);
    if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
  }
  if (p.Tk > 0) {
    if constexpr (DQK + DV <= 256) {
      const int nkb = (p.Tk + 127) / 128;
      hipLaunchKernelGGL((bwd_dkdv_pair_kernel<DQK, DV, DROP>), dim3(nkb * p.B * p.Hkv), dim3(512), 0, st, p);
    } else {
      const int nkb = (p.Tk + 32 * NW_KV - 1) / (32 * NW_KV);
      hipLaunchKernelGGL((bwd_dkdv_kernel<DQK, DV, NW_KV, BQ_KV, DROP>), dim3(nkb * p.B * p.Hkv), dim3(NW_KV * 64), 0,
                         st, p);
    }
    if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
  }
  if (p.Tq > 0) {
    const int rows = p.g * p.Tq;
    const int nrt = (rows + 32 * NW_Q - 1) / (32 * NW_Q);
    hipLaunchKernelGGL((bwd_dq_kernel<DQK, DV, NW_Q, BN_Q, DROP>), dim3(nrt * p.B * p.Hkv), dim3(NW_Q * 64), 0, st, p);
    if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
  }
  return 0;
}

// ---------------------------------------------------------------------------
// 5. Sparse top-k backward, d_qk = d_v = 512 (the values are the pool rows
//    themselves), 64 heads. For query s with gathered rows X (32 per step):
//
//      S^T = X q^T, dP^T = X dO^T         (keys x heads)
//      P = exp(scale S - lse), dS = P (dP - D)
//      dq^T += X^T dS^T                   (scaled at the end)
//      C = [scale dS^T | P^T] [q ; dO]    (keys x columns): the pool rows'
//                                          gradient, key role plus value role
//      dkv[idx] += C                      (fp32 atomics)
//
//    One workgroup per (query, half of the 512 columns), four waves; wave
//    (hg, sl) owns heads 32 hg .. 32 hg + 31. S and dP need all 512 columns:
//    each wave multiplies over columns 256 sl .. 256 sl + 255 and adds its
//    partner's (same heads, other columns) partial through LDS. The two
//    halves of a query repeat S and dP but each adds only its own columns of
//    C, so every (query, slot) adds one 512-column row once. The half's
//    columns of [q ; dO] (128 rows) stay in LDS for the C product, whose B
//    operand comes from transposed reads; its A operand [scale dS | P] is
//    staged key-major in LDS with the rows of each 16-row group permuted into
//    the order the transposed reads deliver ({0-3, 8-11} | {4-7, 12-15}).
//    The atomics of step j are issued at the start of step j + 1, so that
//    the wait for the next rows never waits on them.
// ---------------------------------------------------------------------------
constexpr int kSpD = 512, kSpH = 64, kSpBN = 32;

__global__ void __launch_bounds__(256) bwd_zero_rows_kernel(float* y, int64_t rows, int cols, int64_t st) {
  const int64_t per_row = cols / 4, n = rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / per_row, c = i % per_row;
    *reinterpret_cast<f32x4*>(y + r * st + 4 * c) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_sparse_kernel(const BwdParams p) {
  constexpr int HD = kSpD / 2;                       // columns of one half
  constexpr int CPX = kSpD / 8, CPW = HD / 8, CPY = 2 * kSpH / 8;
  constexpr int WR = 2 * kSpH;                       // rows of [q ; dO]
  constexpr int X_BYTES = kSpBN * kSpD * 2;          // gathered rows
  constexpr int W_BYTES = WR * HD * 2;               // [q ; dO], this half's columns
  constexpr int XB_BYTES = 4 * 2 * 16 * 64 * 4;      // partial S / dP exchange
  constexpr int Y_BYTES = kSpBN * WR * 2;            // [scale dS | P], key-major
  __shared__ __attribute__((aligned(1024))) unsigned char smem[X_BYTES + W_BYTES + XB_BYTES + Y_BYTES + 2 * kSpBN * 4];
  bf16_t* const xt = reinterpret_cast<bf16_t*>(smem);
  bf16_t* const wt = reinterpret_cast<bf16_t*>(smem + X_BYTES);
  float* const xb = reinterpret_cast<float*>(smem + X_BYTES + W_BYTES);
  bf16_t* const yt = reinterpret_cast<bf16_t*>(smem + X_BYTES + W_BYTES + XB_BYTES);
  int32_t* const sidx = reinterpret_cast<int32_t*>(smem + X_BYTES + W_BYTES + XB_BYTES + Y_BYTES);

  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, lh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave & 1, sl = wave >> 1;
  // both halves of a query run on one XCD, next to each other in dispatch order
  const int bi = blockIdx.x;
  const int s = (bi >> 4) * 8 + (bi & 7), e = (bi >> 3) & 1;
  if (s >= p.B) return;
  const int hd = hg * 32 + lq;  // this lane's head
  const int64_t lrow = (int64_t)s * p.H + hd;
  const float lse = p.lse[lrow];
  const float l2 = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
  const float Dr = p.D[lrow];
  const bf16_t* const qs = reinterpret_cast<const bf16_t*>(p.q) + (int64_t)s * p.q_sb;
  const bf16_t* const ds = reinterpret_cast<const bf16_t*>(p.dout) + (int64_t)s * p.do_sb;

  // B operands of S^T and dP^T: this lane's head, columns 256 sl + 16 k + 8 lh ..
  bf16x8 qf[16], dof[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    qf[k] = *reinterpret_cast<const bf16x8*>(qs + (int64_t)hd * p.q_sh + sl * 256 + k * 16 + lh * 8);
    dof[k] = *reinterpret_cast<const bf16x8*>(ds + (int64_t)hd * p.do_sh + sl * 256 + k * 16 + lh * 8);
  }
  // [q ; dO] restricted to this half's columns, row-major (swizzled) in LDS
#pragma unroll
  for (int m = 0; m < WR * CPW / 256; ++m) {
    const int slot = m * 256 + tid, r = slot / CPW, c = slot % CPW;
    const bf16_t* src = r < kSpH ? qs + (int64_t)r * p.q_sh : ds + (int64_t)(r - kSpH) * p.do_sh;
    *reinterpret_cast<u32x4*>(wt + chunk_at<CPW>(r, c)) = *reinterpret_cast<const u32x4*>(src + e * HD + c * 8);
  }

  const int32_t* const ixrow = p.idx + (int64_t)s * p.idx_ss;
  const bf16_t* const pool = reinterpret_cast<const bf16_t*>(p.k);
  const uint32_t xt_s = lds_u32(xt);
  const int nblk = (p.topk + kSpBN - 1) / kSpBN;
  // Block j: lane k (< 32) reads slot j*32 + k; the slots are recorded (-1
  // for a slot past topk or an index outside the pool) and the 32 rows are
  // gathered into LDS, 8 per wave, one 1 KiB row per wave instruction
  // (skipped slots load row 0, never used). Returns the skipped-slot mask.
  auto issue = [&](int j) -> uint32_t {
    const int kk = j * kSpBN + lq;
    const int ix = kk < p.topk ? ixrow[kk] : -1;
    const bool skip = ix < 0 || ix >= p.npool;
    if (wave == 0 && lane < kSpBN) sidx[(j & 1) * kSpBN + lane] = skip ? -1 : ix;
    const uint32_t lane16 = (uint32_t)lane << 4;
#pragma unroll
    for (int m = 0; m < kSpBN / 4; ++m) {
      const int r = wave * (kSpBN / 4) + m;
      const int rix = __builtin_amdgcn_readlane(ix, r);
      const int rowp = (rix >= 0 && rix < p.npool) ? rix : 0;
      dma16(uniform_ptr(pool + (int64_t)rowp * p.k_st), lane16 ^ (uint32_t)(swz<CPX>(r) << 4), xt_s + 1024u * r);
    }
    return (uint32_t)__ballot(skip);
  };

  f32x16 dq[4], C[2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[t][i] = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) C[t][i] = 0.f;

  // C element i of this lane: key lh*4 + 8*(i/4) + i%4, column (2 wave + t)*32 + lq of the half
  auto flush = [&](int j) {
    const int32_t* sx = sidx + (j & 1) * kSpBN;
    float* const base = p.dkv + e * HD + (2 * wave) * 32 + lq;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int n = sx[lh * 4 + 8 * (i >> 2) + (i & 3)];
      if (n >= 0) {
        float* const row = base + (int64_t)n * p.dkv_sn;
        unsafeAtomicAdd(row, C[0][i]);
        unsafeAtomicAdd(row + 32, C[1][i]);
      }
    }
  };

  uint32_t skip_cur = 0;
  if (nblk > 0) skip_cur = issue(0);
  for (int j = 0; j < nblk; ++j) {
    wait_all_loads();
    barrier();  // rows and slots of block j (and [q ; dO]) visible to every wave
    if (j > 0) flush(j - 1);
    // partial S^T, dP^T over this wave's 256 columns (X is the A operand of both)
    f32x16 S, dP;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      S[i] = 0.f;
      dP[i] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bf16x8 a = row_frag<CPX>(xt, lq, sl * 16 + k, lh);
      S = mfma32(a, qf[k], S);
      dP = mfma32(a, dof[k], dP);
    }
    // add the partner's partials (same heads, the other 256 columns)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      *reinterpret_cast<f32x4*>(xb + (((wave * 2 + 0) * 4 + g4) * 64 + lane) * 4) =
          f32x4{S[g4 * 4], S[g4 * 4 + 1], S[g4 * 4 + 2], S[g4 * 4 + 3]};
      *reinterpret_cast<f32x4*>(xb + (((wave * 2 + 1) * 4 + g4) * 64 + lane) * 4) =
          f32x4{dP[g4 * 4], dP[g4 * 4 + 1], dP[g4 * 4 + 2], dP[g4 * 4 + 3]};
    }
    barrier();
    const int pw = wave ^ 2;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(xb + (((pw * 2 + 0) * 4 + g4) * 64 + lane) * 4);
      const f32x4 b = *reinterpret_cast<const f32x4*>(xb + (((pw * 2 + 1) * 4 + g4) * 64 + lane) * 4);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        S[g4 * 4 + q4] += a[q4];
        dP[g4 * 4 + q4] += b[q4];
      }
    }
    // probabilities and dS (skipped slots: P = 0)
    float Pv[16], dSv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = lh * 4 + 8 * (i >> 2) + (i & 3);
      const float pr = ((skip_cur >> key) & 1u) ? 0.f : __builtin_amdgcn_exp2f(fmaf(S[i], p.c, -l2));
      Pv[i] = pr;
      dSv[i] = pr * (dP[i] - Dr);
    }
    // dq^T += X^T dS^T on this wave's four column tiles of the half
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 b = pack8(dSv + ks * 8);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        dq[t] = mfma32(tr_frag<CPX>(xt, ks * 16, e * HD + (4 * sl + t) * 32, lane), b, dq[t]);
    }
    // stage [scale dS | P] key-major: wave sl = 0 writes row hd (scale dS),
    // sl = 1 row 64 + hd (P), at the permuted position of its 16-row group
    {
      const int r = sl == 0 ? hd : kSpH + hd;
      const int q16 = r & 15, pos = (q16 & 3) | ((q16 & 4) << 1) | ((q16 & 8) >> 1);
      const int c = 2 * (r >> 4) + (pos >> 3);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = lh * 4 + 8 * (i >> 2) + (i & 3);
        const float val = sl == 0 ? p.scale * dSv[i] : Pv[i];
        yt[chunk_at<CPY>(key, c) + (pos & 7)] = (bf16_t)val;
      }
    }
    barrier();  // staging complete; the gathered rows and the exchange are free
    if (j + 1 < nblk) skip_cur = issue(j + 1);
    // C = [scale dS | P] [q ; dO] on this wave's two column tiles of the half
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) C[t][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < WR / 16; ++ks) {
      const bf16x8 a = row_frag<CPY>(yt, lq, ks, lh);
#pragma unroll
      for (int t = 0; t < 2; ++t) C[t] = mfma32(a, tr_frag<CPW>(wt, ks * 16, (2 * wave + t) * 32, lane), C[t]);
    }
  }
  if (nblk > 0) flush(nblk - 1);

  bf16_t* const qo = reinterpret_cast<bf16_t*>(p.dq) + (int64_t)s * p.dq_sb + (int64_t)hd * p.dq_sh;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = e * HD + (4 * sl + t) * 32 + g4 * 8 + lh * 4;
      *reinterpret_cast<u32x2*>(qo + d) = u32x2{pack2(dq[t][g4 * 4] * p.scale, dq[t][g4 * 4 + 1] * p.scale),
                                                pack2(dq[t][g4 * 4 + 2] * p.scale, dq[t][g4 * 4 + 3] * p.scale)};
    }
}

// ---------------------------------------------------------------------------
// 6. The forward's extra returns (FA4's widened (out, lse, p, row_max)):
//    p = exp(scale q.k - lse) for the visible keys (0 where masked) and the
//    row maxima of the scaled scores, recomputed from q, k and the forward's
//    lse in a second pass (the fused forward forms neither). One workgroup
//    per 128 query rows of one (b, h); S = Q K^T with Q fragments in
//    registers as the A operand and 32-key K tiles through LDS as the B
//    operand, so that a lane holds one key of 16 rows and each store
//    instruction writes 32 consecutive keys of two rows.
// ---------------------------------------------------------------------------
template <int DQK>
__global__ void __launch_bounds__(256) extras_kernel(const ExtrasParams p) {
  constexpr int NW = 4, BM = 32 * NW, BN = 32, CPK = DQK / 8, KS = DQK / 16;
  constexpr int KT_BYTES = BN * DQK * 2;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * KT_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, lh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_rt = (p.Tq + BM - 1) / BM;
  // the row tiles with the most visible key blocks of every head go first
  // (under a causal mask a tile's work grows with its index)
  const int n_bh = p.B * p.H;
  const int bh = blockIdx.x % n_bh, rt = n_rt - 1 - (int)(blockIdx.x / n_bh);
  const int b = bh / p.H, h = bh % p.H, kvh = h / p.g;
  const int t0 = rt * BM + wave * 32;
  bf16x8 qf[KS];
  {
    const int tq = min(t0 + lq, p.Tq - 1);
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)tq * p.q_st;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + s * 16 + lh * 8);
  }
  // C element r of this lane: row t0 + (r/4)*8 + lh*4 + r%4, key lq of the tile
  const int off = p.Tk - p.Tq;
  const int up = p.causal ? 0 : p.win_right;
  const int64_t lbase = ((int64_t)b * p.H + h) * p.Tq;
  float l2[16], rm[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    // rows past Tq read the last row's lse (clamped, never out of bounds) and
    // write nothing
    const int t = t0 + (r >> 2) * 8 + lh * 4 + (r & 3);
    const float l = p.lse[lbase + min(t, p.Tq - 1)];
    l2[r] = (l == -INFINITY) ? INFINITY : l * kLog2e;
    rm[r] = -INFINITY;
  }
  const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + b * p.k_sb + kvh * p.k_sh;
  float* const pbase = p.p ? p.p + b * p.p_sb + h * p.p_sh : nullptr;
  const uint32_t smem_s = lds_u32(smem);
  const int nb = (p.Tk + BN - 1) / BN;
  // key blocks [jb0, jb1) hold a key some row of the workgroup sees; the
  // blocks outside are masked for all of its rows, so they take no product:
  // p gets zeros there and row_max nothing
  int jb0 = 0, jb1 = nb;
  {
    const int t_lo = rt * BM, t_hi = min(rt * BM + BM - 1, p.Tq - 1);
    if (up >= 0) jb1 = (max(0, min(p.Tk, t_hi + off + up + 1)) + BN - 1) / BN;
    if (p.win_left >= 0) jb0 = min(p.Tk, max(0, t_lo + off - p.win_left)) / BN;
    jb0 = min(jb0, jb1);
  }
  if (jb0 < jb1) dma_tile<CPK, BN, NW>(kbase, p.k_st, jb0 * BN, p.Tk - 1, smem_s + (jb0 & 1) * KT_BYTES, wave, lane);
  for (int j = jb0; j < jb1; ++j) {
    wait_all_loads();
    barrier();
    if (j + 1 < jb1) {
      // the slot address is rebuilt every step (the empty asm), so the per-
      // instruction LDS addresses derived from it are not kept in scalar
      // registers across the loop
      uint32_t slot = smem_s + ((j + 1) & 1) * KT_BYTES;
      asm volatile("" : "+s"(slot));
      dma_tile<CPK, BN, NW>(kbase, p.k_st, (j + 1) * BN, p.Tk - 1, slot, wave, lane);
    }
    const bf16_t* kt = reinterpret_cast<const bf16_t*>(smem + (j & 1) * KT_BYTES);
    f32x16 S;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) S = mfma32(qf[s], row_frag<CPK>(kt, lq, s, lh), S);
    // Row r of this lane is token tl + cr(r) with cr(r) = (r/4)*8 + r%4. With
    // rel = key - (tl + off) the visible keys of row r are the rel in
    // [cr - left, cr + up]; rows from nrow on do not exist. The bounds are
    // rebuilt every step (the empty asm) and tested by sign, so no per-row
    // lane mask is kept across the loop (those would sit in scalar registers).
    const int kk = j * BN + lq;
    int tl = t0 + lh * 4, nrow = p.Tq - tl;
    asm volatile("" : "+v"(tl), "+v"(nrow));
    const int rel = kk - (tl + off);
    const int hi = up >= 0 ? min(up, p.Tk - 1 - kk + rel) : p.Tk - 1 - kk + rel;  // rel <= cr + hi
    const int lo = p.win_left >= 0 ? -p.win_left : -(1 << 30);                     // rel >= cr + lo
    const bool kin = kk < p.Tk;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int cr = (r >> 2) * 8 + (r & 3);
      const int ok = ((cr + hi - rel) | (rel - cr - lo) | (nrow - 1 - cr)) >= 0;  // visible and an existing row
      const float sv = S[r] * p.scale;
      rm[r] = fmaxf(rm[r], ok ? sv : -INFINITY);
      if (pbase != nullptr && kin && cr < nrow)
        pbase[(int64_t)(tl + cr) * p.p_st + kk] = ok ? __builtin_amdgcn_exp2f(fmaf(S[r], p.c, -l2[r])) : 0.f;
    }
  }
  if (pbase != nullptr && (jb0 > 0 || jb1 < nb)) {
    // zeros for the blocks the product loop skipped: lane lq writes key
    // j * BN + lq of this wave's rows tl + cr, the product loop's layout
    const int tl = t0 + lh * 4, nrow = p.Tq - tl;
    for (int j = 0; j < nb; ++j) {
      if (j == jb0) j = jb1;
      if (j >= nb) break;
      const int kk = j * BN + lq;
      if (kk < p.Tk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = (r >> 2) * 8 + (r & 3);
          if (cr < nrow) pbase[(int64_t)(tl + cr) * p.p_st + kk] = 0.f;
        }
      }
    }
  }
  if (p.row_max != nullptr) {
    int tl = t0 + lh * 4;
    asm volatile("" : "+v"(tl));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = rm[r];
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
      const int t = tl + (r >> 2) * 8 + (r & 3);
      if (lq == 0 && t < p.Tq) p.row_max[lbase + t] = v;
    }
  }
}

template <int DQK>
int launch_extras_d(const ExtrasParams& p, void* stream) {
  const int n_rt = (p.Tq + 127) / 128;
  const int64_t grid = (int64_t)p.B * p.H * n_rt;
  if (grid == 0) return 0;
  hipLaunchKernelGGL(extras_kernel<DQK>, dim3((unsigned)grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

}  // namespace

bool bwd_supported(int d_qk, int d_v) {
  return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128) ||
         (d_qk == 256 && d_v == 256) || (d_qk == 512 && d_v == 512);
}

bool dropout_supported(int d_qk, int d_v) { return bwd_supported(d_qk, d_v); }

int bwd_head_splits(int B, int Hkv, int g, int Tk, int d_qk, int d_v) {
  if (d_qk != d_v || (d_qk != 256 && d_qk != 512) || Tk <= 0 || g <= 1) return 1;
  const int bnk = d_qk == 512 ? 32 : 64;  // keys per dK/dV workgroup
  const int64_t base = (int64_t)B * Hkv * ((Tk + bnk - 1) / bnk);
  // one workgroup fits a CU: ask for about three per CU of the 256 so that the
  // short causal key blocks fill in behind the long ones; at most 16 splits
  // (the partials' traffic grows with their number). Measured on the MQA
  // d512 shape (44 key blocks): 8 splits 12% and 12 splits 2% slower than
  // 16; 32 the same time with twice the workspace
  if (base >= 512) return 1;
  return (int)std::min<int64_t>({(int64_t)g, 16, (768 + base - 1) / base});
}

int launch_bwd(const BwdParams& p, int d_qk, int d_v, void* stream) {
  const bool drop = p.keep != nullptr;
  if (d_qk == 64 && d_v == 64) return drop ? launch_bwd_cfg<64, 64, true>(p, stream) : launch_bwd_cfg<64, 64, false>(p, stream);
  if (d_qk == 128 && d_v == 128)
    return drop ? launch_bwd_cfg<128, 128, true>(p, stream) : launch_bwd_cfg<128, 128, false>(p, stream);
  if (d_qk == 192 && d_v == 128)
    return drop ? launch_bwd_cfg<192, 128, true>(p, stream) : launch_bwd_cfg<192, 128, false>(p, stream);
  if (d_qk == 256 && d_v == 256)
    return drop ? launch_bwd_wide<256, true>(p, stream) : launch_bwd_wide<256, false>(p, stream);
  if (d_qk == 512 && d_v == 512)
    return drop ? launch_bwd_wide<512, true>(p, stream) : launch_bwd_wide<512, false>(p, stream);
  return -1;
}

int launch_bwd_sparse(const BwdParams& p, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t n4 = (int64_t)p.npool * (kSpD / 4);
  if (n4 > 0) {
    const int64_t grid = std::min<int64_t>((n4 + 255) / 256, 8192);
    hipLaunchKernelGGL(bwd_zero_rows_kernel, dim3((unsigned)grid), dim3(256), 0, st, p.dkv, (int64_t)p.npool, kSpD,
                       p.dkv_sn);
    if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
  }
  const int64_t R = (int64_t)p.B * p.H;
  if (R > 0) {
    hipLaunchKernelGGL(bwd_dot_kernel<kSpD>, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, st, p);
    if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
    if (p.sinks != nullptr && p.dsinks != nullptr) {
      hipLaunchKernelGGL(bwd_dsink_kernel, dim3(p.H), dim3(256), 0, st, p);
      if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
    }
    hipLaunchKernelGGL(bwd_sparse_kernel, dim3((unsigned)(((p.B + 7) / 8) * 16)), dim3(256), 0, st, p);
    if (hipPeekAtLastError() != hipSuccess) return (int)hipGetLastError();
  }
  return 0;
}

bool extras_supported(int d_qk) { return d_qk == 64 || d_qk == 128 || d_qk == 192 || d_qk == 256 || d_qk == 512; }

int launch_extras(const ExtrasParams& p, int d_qk, void* stream) {
  switch (d_qk) {
    case 64: return launch_extras_d<64>(p, stream);
    case 128: return launch_extras_d<128>(p, stream);
    case 192: return launch_extras_d<192>(p, stream);
    case 256: return launch_extras_d<256>(p, stream);
    case 512: return launch_extras_d<512>(p, stream);
    default: return -1;
  }
}

int launch_fwd_dropout(const BwdParams& p, int d_qk, int d_v, void* stream) {
  const int64_t n_rt = ((int64_t)p.g * p.Tq + 127) / 128;
  const int64_t grid = n_rt * p.B * p.Hkv;
  if (grid == 0) return 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (d_qk == 64 && d_v == 64)
    hipLaunchKernelGGL((fwd_dropout_kernel<64, 64>), dim3((unsigned)grid), dim3(256), 0, st, p);
  else if (d_qk == 128 && d_v == 128)
    hipLaunchKernelGGL((fwd_dropout_kernel<128, 128>), dim3((unsigned)grid), dim3(256), 0, st, p);
  else if (d_qk == 192 && d_v == 128)
    hipLaunchKernelGGL((fwd_dropout_kernel<192, 128>), dim3((unsigned)grid), dim3(256), 0, st, p);
  else if (d_qk == 256 && d_v == 256)
    hipLaunchKernelGGL((fwd_dropout_kernel<256, 256>), dim3((unsigned)grid), dim3(256), 0, st, p);
  else
    return -1;  // (512-wide heads take the mask inside the fused forward)
  return (int)hipGetLastError();
}

int launch_sparse_fp8(const SpFp8Params& p, void* stream) {
  if (p.Sq == 0) return 0;
  hipLaunchKernelGGL(sparse_fp8_kernel, dim3((unsigned)p.Sq, (unsigned)p.n_splits), dim3(512), 0,
                     reinterpret_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

}  // namespace attn
