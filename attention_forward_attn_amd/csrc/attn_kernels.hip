// Fused attention forward for AMD CDNA4 (gfx950 / MI355X).
//
// One workgroup owns a block of query rows and streams the keys through LDS:
//
//   S^T = K Q^T      on v_mfma_f32_32x32x16_bf16 (fp32 accumulate)
//   online softmax   row max / row sum kept in registers, exp2 with the
//                    scale*log2(e) factor folded into one FMA, lazy rescale
//   O^T += V^T P^T   on the same MFMA, P taken straight from the S^T
//                    accumulators after bf16 packing
//
// The scores are computed transposed (keys along the MFMA M dimension,
// queries along N) so that every lane owns exactly one query row: lane l holds
// query column l%32 and 16 of the 32 keys of a 32x32 tile, the other 16 being
// in lane l^32. Row max and row sum are in-lane reductions plus one exchange
// with the partner half-wave (v_permlane32_swap), the rescale of the output
// accumulator is a per-lane multiply, and the S^T accumulator is already laid
// out as the B operand that O^T = V^T P^T needs (no shuffle of P).
//
// Two kernel families live here:
//
//   attn_fwd_dma_kernel (every bf16 path: dense, folded GQA/MQA, split-KV,
//     windows, packed batches, two-part MLA rows, sparse top-k). K and V tiles
//     go from global memory straight into LDS with global_load_lds_dwordx4
//     (16 bytes per lane, no staging registers); the bank-conflict swizzle is
//     applied on the global side, and the V^T operands of the PV product are
//     read from the row-major V tile with ds_read_b64_tr_b16 (no transposed
//     copy of V exists). Loads are issued from inline asm and waited for with
//     exact per-wave vmcnt counts and plain s_barriers. Narrow heads (64, 128,
//     192) run two wave groups per workgroup that alternate their MFMA half
//     (S and PV) and their softmax half on each SIMD; 256- and 512-wide heads
//     split d over DS waves of a query group and sum the partial scores
//     through LDS; the 512-wide instance also comes with the caller's dropout
//     keep mask applied inside (DROP). Described in detail above the kernel.
//
//   attn_fwd_kernel (fp32 inputs only, the tiny workload): the first kernel of
//     this library, register-staged: 16-byte global loads into registers, V
//     transposed in registers (4 keys x 8 columns per thread) and stored to
//     LDS as V^T, each fp32 q/k value split into a bf16 hi + lo pair so that
//     S = hi*hi + hi*lo + lo*hi keeps ~16 bits on the bf16 MFMA.
//
// GQA/MQA: the query rows of one (batch, kv head) are the folded view
// [g*Tq, d] of q[B,H,Tq,d] with kv-major heads (ArcFlash pull request,
// "What rung 0 does"): pure index arithmetic, nothing is copied. The bf16
// kernels order the folded rows token-major (row t*g + head) so that a causal
// tile spans few tokens.
//
// Sparse top-k (TensorRT-LLM pull request 22028, "Description"): the rows of a
// workgroup are the heads of one query; the keys are the pool rows named by
// the query's index list, gathered into the same LDS tiles. The value rows are
// the first d_v columns of the same gathered rows, so every gathered row is
// read from memory once and serves both products.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_params.h"

namespace attn {
namespace {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// value held by lane l ^ 32
// v_permlane32_swap leaves lanes 0-31 of both halves in one register and
// lanes 32-63 in the other, so one VALU op combines the two row halves held
// by lanes l and l ^ 32 (no LDS round trip).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Note: reinterpret single vector elements with __uint_as_float, never with
// __builtin_bit_cast(float, vec[i]) -- this compiler lowers the latter to a
// read of element 0 of the vector.

// split 8 floats into high and low bfloat16 parts: x ~= hi + lo with ~16 bits
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16_t h0 = (bf16_t)x[2 * i], h1 = (bf16_t)x[2 * i + 1];
    float r0 = x[2 * i] - (float)h0, r1 = x[2 * i + 1] - (float)h1;
    h[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    l[i] = pack_bf16x2(r0, r1);
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// position of key-quad kq (4 keys) inside a V^T row: quads {0,2,1,3} of each 16-key group
__device__ __forceinline__ int vquad_pos(int kq) {
  const int q = kq & 3;
  return (kq & ~3) | ((q & 1) << 1) | (q >> 1);
}

template <int DQK, int DV, int QT, int DS, int NW, int BN, bool F32, bool SPARSE>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int NQG = NW / DS;           // query groups per workgroup
  static constexpr int BM = NQG * QT * 32;      // query rows per workgroup
  static constexpr int DQW = DQK / DS;          // d_qk columns per wave
  static constexpr int DVW = DV / DS;           // d_v columns per wave
  static constexpr int KS = DQW / 16;           // MFMA k-steps of S per wave
  static constexpr int MT = BN / 32;            // 32-key tiles per block
  static constexpr int DT = DVW / 32;           // 32-column output tiles per wave
  static constexpr int PKS = BN / 16;           // MFMA k-steps of PV
  static constexpr int K_LD = DQK + 8;          // K row stride in LDS (elements)
  static constexpr int V_LD = BN + 4;           // V^T row stride in LDS (elements)
  static constexpr int NSPLIT = F32 ? 2 : 1;    // hi/lo bf16 parts for fp32 inputs
  static constexpr int K_ELEMS = BN * K_LD;
  static constexpr int V_ELEMS = DV * V_LD;
  static constexpr int STAGE_ELEMS = NSPLIT * (K_ELEMS + V_ELEMS);
  static constexpr int SX_FLOATS = (DS > 1) ? NW * QT * MT * 16 * 64 : 0;
  static constexpr int FLAG_BYTES = SPARSE ? 2 * BN : 0;
  static constexpr int LDS_BYTES = 2 * STAGE_ELEMS * 2 + SX_FLOATS * 4 + FLAG_BYTES;
  // dense K tile loading: 8-element chunks, consecutive threads along a row
  static constexpr int KCH = BN * DQK / 8;
  static constexpr int KCH_PT = (KCH + NT - 1) / NT;
  // V loading (and all sparse loading): units of 4 keys x 8 columns
  static constexpr int UCOLS = SPARSE ? DQK : DV;
  static constexpr int VU = (BN / 4) * (UCOLS / 8);
  static constexpr int VU_PT = (VU + NT - 1) / NT;
  static constexpr int WORDS = F32 ? 8 : 4;     // 32-bit words per 8-element chunk
  static_assert(DQK % (16 * DS) == 0 && DV % (32 * DS) == 0, "head dims must tile");
  static_assert(BN % 32 == 0, "BN must be a multiple of 32");
  static_assert(!(SPARSE && F32), "sparse path is bf16 only");
  static_assert(!SPARSE || DV <= DQK, "sparse value columns are a prefix of the row");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
};

template <int DQK, int DV, int QT, int DS, int NW, int BN, bool F32, bool SPARSE>
__global__ void __launch_bounds__(NW * 64)
attn_fwd_kernel(const KernelParams p) {
  using C = Cfg<DQK, DV, QT, DS, NW, BN, F32, SPARSE>;
  using in_t = typename std::conditional<F32, float, bf16_t>::type;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS_BYTES];
  bf16_t* const lds = reinterpret_cast<bf16_t*>(smem);
  float* const sx = reinterpret_cast<float*>(smem + 2 * C::STAGE_ELEMS * 2);
  unsigned char* const flags = smem + 2 * C::STAGE_ELEMS * 2 + C::SX_FLOATS * 4;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, lh = lane >> 5;
  const int qg = wave / DS, dsi = wave % DS;

  // ---------------------------------------------------------------- tile
  int b = 0, kvh = 0, f0 = 0, nrows = 0, t_lo = 0, t_hi = 0, sq = 0;
  if constexpr (SPARSE) {
    sq = blockIdx.x;
    nrows = p.H;
  } else {
    const int tile = blockIdx.x;
    if (p.aligned) {
      // largest causal row blocks first (longest-processing-time order)
      const int per_tb = p.n_groups * p.g;
      const int tb = (p.tiles_per_head - 1) - tile / per_tb;
      const int rest = tile % per_tb;
      const int grp = rest / p.g, hl = rest % p.g;
      b = grp / p.Hkv;
      kvh = grp % p.Hkv;
      const int t0 = tb * C::BM;
      f0 = hl * p.Tq + t0;
      nrows = min(C::BM, p.Tq - t0);
      t_lo = t0;
      t_hi = t0 + nrows - 1;
    } else {
      const int grp = tile / p.tiles_per_group;
      f0 = (tile % p.tiles_per_group) * C::BM;
      nrows = min(C::BM, p.g * p.Tq - f0);
      b = grp / p.Hkv;
      kvh = grp % p.Hkv;
      const int tf = f0 % p.Tq;
      if (nrows >= p.Tq || tf + nrows > p.Tq) {
        t_lo = 0;
        t_hi = p.Tq - 1;
      } else {
        t_lo = tf;
        t_hi = tf + nrows - 1;
      }
    }
  }

  // keys [0, kend) are needed; below kfull no row of the tile is masked
  int kend = p.Tk, kfull = p.Tk;
  if (!SPARSE && p.causal) {
    const int off = p.Tk - p.Tq;
    kend = min(p.Tk, max(0, t_hi + off + 1));
    kfull = min(p.Tk, max(0, t_lo + off + 1));
  }
  const int nblk = (kend + BN - 1) / BN;

  // ---------------------------------------------------------------- rows of this lane
  bool row_ok[QT];
  int row_lim[QT];        // last visible key (dense)
  int row_h[QT];
  int64_t q_off[QT], o_off[QT], l_off[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = (qg * QT + qt) * 32 + lq;
    row_ok[qt] = r < nrows;
    const int rr = row_ok[qt] ? r : 0;
    if constexpr (SPARSE) {
      row_h[qt] = rr;
      row_lim[qt] = p.Tk - 1;
      q_off[qt] = (int64_t)sq * p.q_sb + (int64_t)rr * p.q_sh;
      o_off[qt] = (int64_t)sq * p.o_sb + (int64_t)rr * p.o_sh;
      l_off[qt] = (int64_t)sq * p.H + rr;
    } else {
      const int f = f0 + rr;
      const int h = kvh * p.g + f / p.Tq;
      const int t = f % p.Tq;
      row_h[qt] = h;
      row_lim[qt] = p.causal ? min(p.Tk - 1, t + p.Tk - p.Tq) : p.Tk - 1;
      q_off[qt] = (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)t * p.q_st;
      o_off[qt] = (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)t * p.o_st;
      l_off[qt] = ((int64_t)b * p.H + h) * p.Tq + t;
    }
  }

  // ---------------------------------------------------------------- Q fragments (B operand of S^T)
  bf16x8 qf[QT][C::KS];
  bf16x8 qlo[F32 ? QT : 1][F32 ? C::KS : 1];
  {
    const in_t* qb = reinterpret_cast<const in_t*>(p.q);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const int d0 = dsi * C::DQW + s * 16 + lh * 8;
        if constexpr (F32) {
          float x[8];
          if (row_ok[qt]) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(qb + q_off[qt] + d0);
            const f32x4 c = *reinterpret_cast<const f32x4*>(qb + q_off[qt] + d0 + 4);
            x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
            x[4] = c[0]; x[5] = c[1]; x[6] = c[2]; x[7] = c[3];
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.f;
          }
          u32x4 hi, lo;
          split8(x, hi, lo);
          qf[qt][s] = as_bf16x8(hi);
          qlo[qt][s] = as_bf16x8(lo);
        } else {
          u32x4 w = {0u, 0u, 0u, 0u};
          if (row_ok[qt]) w = *reinterpret_cast<const u32x4*>(qb + q_off[qt] + d0);
          qf[qt][s] = as_bf16x8(w);
        }
      }
    }
  }

  // ---------------------------------------------------------------- tile loader
  const in_t* kbase;
  const in_t* vbase;
  if constexpr (SPARSE) {
    kbase = reinterpret_cast<const in_t*>(p.k);
    vbase = kbase;
  } else {
    kbase = reinterpret_cast<const in_t*>(p.k) + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
    vbase = reinterpret_cast<const in_t*>(p.v) + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh;
  }
  const int32_t* idx_row = SPARSE ? p.idx + (int64_t)sq * p.idx_ss : nullptr;

  u32x4 kst[SPARSE ? 1 : C::KCH_PT][C::WORDS / 4];
  u32x4 vst[C::VU_PT][4][C::WORDS / 4];
  int32_t sidx[4];        // sparse: pool rows of this thread's 4 keys for the next load
  uint32_t svalid = 0;    // sparse: validity bits of the staged keys

  auto load_idx = [&](int blk) {
    // this thread's key quad is the same for all its units (unit stride NT is a multiple of BN/4)
    const int kq = tid % (BN / 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = blk * BN + 4 * kq + r;
      sidx[r] = (kk < p.Tk) ? idx_row[kk] : -1;
    }
  };

  auto load_tile = [&](int blk) {
    const int key0 = blk * BN;
    if constexpr (!SPARSE) {
#pragma unroll
      for (int i = 0; i < C::KCH_PT; ++i) {
        const int c = tid + i * C::NT;
        const int key = c / (DQK / 8), dc = c % (DQK / 8);
        const int kk = key0 + key;
        const bool ok = (c < C::KCH) && (kk < kend);
        const in_t* src = kbase + (int64_t)kk * p.k_st + dc * 8;
#pragma unroll
        for (int w = 0; w < C::WORDS / 4; ++w)
          kst[i][w] = ok ? *reinterpret_cast<const u32x4*>(src + w * 4) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < C::VU_PT; ++i) {
        const int u = tid + i * C::NT;
        const int kq = u % (BN / 4), dc = u / (BN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = key0 + 4 * kq + r;
          const bool ok = (u < C::VU) && (kk < kend);
          const in_t* src = vbase + (int64_t)kk * p.v_st + dc * 8;
#pragma unroll
          for (int w = 0; w < C::WORDS / 4; ++w)
            vst[i][r][w] = ok ? *reinterpret_cast<const u32x4*>(src + w * 4) : u32x4{0u, 0u, 0u, 0u};
        }
      }
    } else {
      (void)key0;
      uint32_t vb = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) vb |= (sidx[r] >= 0 && sidx[r] < p.npool) ? (1u << r) : 0u;
      svalid = vb;
#pragma unroll
      for (int i = 0; i < C::VU_PT; ++i) {
        const int u = tid + i * C::NT;
        const int dc = u / (BN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = (u < C::VU) && ((vb >> r) & 1u);
          const in_t* src = kbase + (int64_t)(ok ? sidx[r] : 0) * p.k_st + dc * 8;
          vst[i][r][0] = ok ? *reinterpret_cast<const u32x4*>(src) : u32x4{0u, 0u, 0u, 0u};
        }
      }
      if (blk + 1 < nblk) load_idx(blk + 1);
    }
  };

  auto store_tile = [&](int buf) {
    bf16_t* Kb = lds + buf * C::STAGE_ELEMS;
    bf16_t* Vb = Kb + C::NSPLIT * C::K_ELEMS;
    if constexpr (!SPARSE) {
#pragma unroll
      for (int i = 0; i < C::KCH_PT; ++i) {
        const int c = tid + i * C::NT;
        if (c < C::KCH) {
          const int key = c / (DQK / 8), dc = c % (DQK / 8);
          bf16_t* dst = Kb + key * C::K_LD + dc * 8;
          if constexpr (F32) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(kst[i][e / 4][e % 4]);
            u32x4 hi, lo;
            split8(x, hi, lo);
            *reinterpret_cast<u32x4*>(dst) = hi;
            *reinterpret_cast<u32x4*>(dst + C::K_ELEMS) = lo;
          } else {
            *reinterpret_cast<u32x4*>(dst) = kst[i][0];
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::VU_PT; ++i) {
      const int u = tid + i * C::NT;
      if (u < C::VU) {
        const int kq = u % (BN / 4), dc = u / (BN / 4);
        // rows as bf16 words: hv[part][r] = 4 words (8 elements) of key r
        u32x4 hv[C::NSPLIT][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (F32) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(vst[i][r][e / 4][e % 4]);
            split8(x, hv[0][r], hv[C::NSPLIT - 1][r]);
          } else {
            hv[0][r] = vst[i][r][0];
          }
        }
        if constexpr (SPARSE) {
          // row-major K tile from the same gathered rows
#pragma unroll
          for (int r = 0; r < 4; ++r)
            *reinterpret_cast<u32x4*>(Kb + (4 * kq + r) * C::K_LD + dc * 8) = hv[0][r];
        }
        if (!SPARSE || dc < DV / 8) {
          // transpose 4 keys x 8 columns into 8 V^T rows of 4 keys
          const int col = vquad_pos(kq) * 4;
#pragma unroll
          for (int part = 0; part < C::NSPLIT; ++part) {
            bf16_t* vdst = Vb + part * C::V_ELEMS + (dc * 8) * C::V_LD + col;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int w = j >> 1;
              uint32_t x0, x1;
              if (j & 1) {
                x0 = (hv[part][0][w] >> 16) | (hv[part][1][w] & 0xffff0000u);
                x1 = (hv[part][2][w] >> 16) | (hv[part][3][w] & 0xffff0000u);
              } else {
                x0 = (hv[part][0][w] & 0xffffu) | (hv[part][1][w] << 16);
                x1 = (hv[part][2][w] & 0xffffu) | (hv[part][3][w] << 16);
              }
              *reinterpret_cast<u32x2*>(vdst + j * C::V_LD) = u32x2{x0, x1};
            }
          }
        }
      }
    }
    if constexpr (SPARSE) {
      if (tid < BN / 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) flags[buf * BN + 4 * tid + r] = (svalid >> r) & 1u;
      }
    }
  };

  // ---------------------------------------------------------------- state
  f32x16 acc[QT][C::DT];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[qt][dt][i] = 0.f;
  }

  if (nblk > 0) {
    if constexpr (SPARSE) load_idx(0);
    load_tile(0);
    store_tile(0);
    if (nblk > 1) load_tile(1);
  }

  for (int blk = 0; blk < nblk; ++blk) {
    __syncthreads();
    const int buf = blk & 1;
    const bf16_t* Kb = lds + buf * C::STAGE_ELEMS;
    const bf16_t* Vb = Kb + C::NSPLIT * C::K_ELEMS;
    const int key0 = blk * BN;

    // ---- S^T = K Q^T (partial over this wave's d_qk columns)
    f32x16 S[QT][C::MT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[qt][mt][i] = 0.f;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const int off = (mt * 32 + lq) * C::K_LD + dsi * C::DQW + s * 16 + lh * 8;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + off);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) S[qt][mt] = mfma32(a, qf[qt][s], S[qt][mt]);
        if constexpr (F32) {
          const bf16x8 alo = *reinterpret_cast<const bf16x8*>(Kb + C::K_ELEMS + off);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            S[qt][mt] = mfma32(alo, qf[qt][s], S[qt][mt]);
            S[qt][mt] = mfma32(a, qlo[qt][s], S[qt][mt]);
          }
        }
      }
    }

    // ---- sum the partial scores of the DS waves sharing these rows
    if constexpr (DS > 1) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float* dst = sx + ((((wave * QT + qt) * C::MT + mt) * 4 + g4) * 64 + lane) * 4;
            *reinterpret_cast<f32x4*>(dst) =
                f32x4{S[qt][mt][g4 * 4], S[qt][mt][g4 * 4 + 1], S[qt][mt][g4 * 4 + 2], S[qt][mt][g4 * 4 + 3]};
          }
      __syncthreads();
#pragma unroll
      for (int o = 1; o < DS; ++o) {
        const int w2 = qg * DS + (dsi + o) % DS;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const float* src = sx + ((((w2 * QT + qt) * C::MT + mt) * 4 + g4) * 64 + lane) * 4;
              const f32x4 v = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
              for (int e = 0; e < 4; ++e) S[qt][mt][g4 * 4 + e] += v[e];
            }
      }
    }

    // ---- masks: causal / ragged tail (dense) or skipped indices (sparse)
    if constexpr (SPARSE) {
      const unsigned char* fl = flags + buf * BN;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const uint32_t f4 = *reinterpret_cast<const uint32_t*>(fl + mt * 32 + g4 * 8 + lh * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (((f4 >> (8 * e)) & 0xffu) == 0u)
#pragma unroll
              for (int qt = 0; qt < QT; ++qt) S[qt][mt][g4 * 4 + e] = -INFINITY;
        }
    } else {
      if (key0 + BN > kfull) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = key0 + mt * 32 + (i >> 2) * 8 + lh * 4 + (i & 3);
              if (key > row_lim[qt]) S[qt][mt][i] = -INFINITY;
            }
      }
    }

    // ---- online softmax (base 2, scale folded into the FMA)
    bf16x8 pb[QT][C::PKS];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[qt][mt][i]);
      mx = halves_max(mx);
      const float mnew = fmaxf(m_run[qt], mx);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f((m_run[qt] - muse) * p.c);
      const float mc = muse * p.c;
      float rs = 0.f;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(S[qt][mt][i], p.c, -mc));
          S[qt][mt][i] = e;
          rs += e;
        }
      l_run[qt] = l_run[qt] * alpha + rs;
      m_run[qt] = mnew;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[qt][dt][i] *= alpha;
#pragma unroll
      for (int ks = 0; ks < C::PKS; ++ks) {
        const int mt = ks >> 1, base = (ks & 1) * 8;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(S[qt][mt][base + 2 * e], S[qt][mt][base + 2 * e + 1]);
        pb[qt][ks] = as_bf16x8(w);
      }
    }

    // ---- O^T += V^T P^T over this wave's d_v columns
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int ks = 0; ks < C::PKS; ++ks) {
        const int off = (dsi * C::DVW + dt * 32 + lq) * C::V_LD + ks * 16 + lh * 8;
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(Vb + off);
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(Vb + off + 4);
        const bf16x8 a = as_bf16x8(u32x4{a0[0], a0[1], a1[0], a1[1]});
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) acc[qt][dt] = mfma32(a, pb[qt][ks], acc[qt][dt]);
        if constexpr (F32) {
          const u32x2 b0 = *reinterpret_cast<const u32x2*>(Vb + C::V_ELEMS + off);
          const u32x2 b1 = *reinterpret_cast<const u32x2*>(Vb + C::V_ELEMS + off + 4);
          const bf16x8 alo = as_bf16x8(u32x4{b0[0], b0[1], b1[0], b1[1]});
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) acc[qt][dt] = mfma32(alo, pb[qt][ks], acc[qt][dt]);
        }
      }
    }

    // ---- stage the next tile, prefetch the one after
    if (blk + 1 < nblk) {
      store_tile(buf ^ 1);
      if (blk + 2 < nblk) load_tile(blk + 2);
    }
  }

  // ---------------------------------------------------------------- epilogue
  in_t* ob = reinterpret_cast<in_t*>(p.out);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = halves_sum(l_run[qt]);
    const float ms = (m_run[qt] == -INFINITY) ? -INFINITY : m_run[qt] * p.scale;  // natural units
    float inv, lse;
    if (p.sinks != nullptr) {
      const float sk = p.sinks[row_h[qt]];
      const float M = fmaxf(ms, sk);
      if (M == -INFINITY) {
        inv = 0.f;
        lse = -INFINITY;
      } else {
        const float fac = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((ms - M) * kLog2e);
        const float es = (sk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((sk - M) * kLog2e);
        const float den = lt * fac + es;
        inv = den > 0.f ? fac / den : 0.f;
        lse = den > 0.f ? M + __builtin_amdgcn_logf(den) * kLn2 : -INFINITY;
      }
    } else {
      inv = lt > 0.f ? 1.f / lt : 0.f;
      lse = lt > 0.f ? ms + __builtin_amdgcn_logf(lt) * kLn2 : -INFINITY;
    }
    if (row_ok[qt]) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = dsi * C::DVW + dt * 32 + g4 * 8 + lh * 4;
          const float v0 = acc[qt][dt][g4 * 4] * inv, v1 = acc[qt][dt][g4 * 4 + 1] * inv;
          const float v2 = acc[qt][dt][g4 * 4 + 2] * inv, v3 = acc[qt][dt][g4 * 4 + 3] * inv;
          if constexpr (F32) {
            *reinterpret_cast<f32x4*>(ob + o_off[qt] + d) = f32x4{v0, v1, v2, v3};
          } else {
            *reinterpret_cast<u32x2*>(ob + o_off[qt] + d) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          }
        }
      }
      if (lh == 0 && dsi == 0) p.lse[l_off[qt]] = lse;
    }
  }
}

// ===========================================================================
// bf16 kernel family with direct-to-LDS staging.
//
// K and V tiles travel from global memory straight into LDS with
// global_load_lds_dwordx4 (16 bytes per lane, no staging registers, no LDS
// store instructions). A wave instruction fills 64 consecutive 16-byte LDS
// slots, so the bank-conflict swizzle is applied on the global side: the lane
// that owns slot (row r, physical chunk p) fetches logical chunk p ^ swz(r).
// V^T operands of the PV product are read from the row-major V tile with
// ds_read_b64_tr_b16, which transposes 4x16 blocks of 16-bit elements across
// each 16-lane group; no transposed copy of V exists. In the sparse path the
// gathered pool rows form one tile that serves both products (V == K).
//
// The direct-to-LDS loads are issued from inline asm so that the compiler
// does not insert a conservative vmcnt(0) before every LDS read; the kernel
// waits for exactly the loads of the tile it is about to use and synchronises
// with a plain s_barrier. With NSTAGE = 3 the loads of tile i+2 are in flight
// while tile i is multiplied and one barrier per tile suffices.
//
// Online softmax with a lazy rescale: the running row max only moves when a
// new score exceeds it by more than kRescaleLog2 (in log2 units), so the
// output accumulator is rescaled on the first key blocks and almost never
// afterwards; exp2 arguments stay <= kRescaleLog2, far from fp32 overflow.
// ===========================================================================

constexpr float kRescaleLog2 = 8.f;

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;
#ifndef ATTN_LDS_PREFETCH
#define ATTN_LDS_PREFETCH 4
#endif
constexpr int kPrefetch = ATTN_LDS_PREFETCH;  // MFMA operands read from LDS ahead of use

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory into LDS at m0 + 16 * lane, read
// from a wave-uniform base plus a per-lane 32-bit byte offset (the SGPR-base
// form of the instruction: no 64-bit address arithmetic per load).
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               ::"v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// The same with a full 64-bit address per lane (no scalar base): the lanes of
// one instruction may read from two different tensors.
__device__ __forceinline__ void dma16v(uint64_t addr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(addr), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// a pointer that is the same in every lane, moved to scalar registers
__device__ __forceinline__ const void* uniform_ptr(const void* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// vmcnt wait with a wave-uniform count (0..31)
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 17: wait_vmcnt<17>(); break;
    case 18: wait_vmcnt<18>(); break;
    case 19: wait_vmcnt<19>(); break;
    case 20: wait_vmcnt<20>(); break;
    case 21: wait_vmcnt<21>(); break;
    case 22: wait_vmcnt<22>(); break;
    case 23: wait_vmcnt<23>(); break;
    case 24: wait_vmcnt<24>(); break;
    case 25: wait_vmcnt<25>(); break;
    case 26: wait_vmcnt<26>(); break;
    case 27: wait_vmcnt<27>(); break;
    case 28: wait_vmcnt<28>(); break;
    case 29: wait_vmcnt<29>(); break;
    case 30: wait_vmcnt<30>(); break;
    default: wait_vmcnt<31>(); break;
  }
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Chunk swizzle of a tile row with CPR 16-byte chunks. LDS serves 256 bytes
// (16 chunks, 64 banks) per cycle. Rows whose length is a multiple of 256
// bytes start on the same bank, so the swizzle is a 4-bit XOR: 16 consecutive
// rows send one logical chunk to 16 distinct bank groups (A-operand reads of
// K), and rows 4k..4k+3 send an aligned 4-chunk group to 4 distinct groups
// (transposed V reads). Rows of 128 + 256n bytes alternate between the two
// halves of the banks, so a 3-bit XOR inside aligned 8-chunk groups gives the
// same two properties and keeps every chunk inside the row.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  static_assert(CPR % 8 == 0, "rows are whole 8-chunk groups");
  if constexpr (CPR % 16 == 0)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// XK (one wave group, DS > 1, dense): the K ring has one slot more than the
// V ring and no separate score-exchange buffer; the partial scores of key
// block j are exchanged in the K slot block j was read from, once every wave
// has read it. The LDS saved keeps a second K block in flight.
template <int DQK, int DV, int DS, int NW, int BN, int NBUF, bool SPARSE, bool PINGPONG, bool XK = false>
struct DCfg {
  static constexpr int NT = NW * 64;
  static constexpr int NQG = NW / DS;
  static constexpr int BM = NQG * 32;
  static constexpr int DQW = DQK / DS;
  static constexpr int DVW = DV / DS;
  static constexpr int KS = DQW / 16;
  static constexpr int MT = BN / 32;
  static constexpr int DT = DVW / 32;
  static constexpr int PKS = BN / 16;
  static constexpr int CPRK = DQK / 8;
  static constexpr int CPRV = DV / 8;
  static constexpr int VLD = SPARSE ? DQK : DV;  // row length of the tile V is read from
  static constexpr int K_ELEMS = BN * DQK;
  static constexpr int V_ELEMS = SPARSE ? 0 : BN * DV;
  // Two wave groups (one wave of each per SIMD with 8 waves) or one.
  static constexpr bool PP = PINGPONG;
  // With two groups, K block j is read in the two halves of key step j and
  // V block j in the two halves of step j+1; with one group both are read in
  // step j. K block j+KD (V block j+VD) is loaded while step j runs, into the
  // ring slot of a block nobody reads any more.
  static constexpr int NBK = XK ? NBUF + 1 : NBUF;  // K ring slots
  static constexpr int KD = XK ? NBK - 1 : (PP && SPARSE) ? NBUF - 2 : NBUF - 1;
  static constexpr int VD = PP ? NBUF - 2 : NBUF - 1;
  static constexpr int NIK = BN * CPRK / 64;     // wave instructions per K tile
  static constexpr int NIV = SPARSE ? 0 : BN * CPRV / 64;
  static constexpr int SX_PART_BYTES = NW * MT * 16 * 64 * 4;  // partial scores of one key block
  static constexpr int SX_BYTES = (DS > 1 && !XK) ? SX_PART_BYTES : 0;
  static constexpr int IDX_CAP = SPARSE ? 4096 : 0;
  static constexpr int KRING_BYTES = NBK * K_ELEMS * 2;
  static constexpr int VRING_BYTES = NBUF * V_ELEMS * 2;
  static constexpr int LDS_BYTES = KRING_BYTES + VRING_BYTES + SX_BYTES + IDX_CAP * 4;
  static_assert(KD >= 1, "at least one key step of prefetch");
  static_assert(!XK || (!PP && !SPARSE && DS > 1 && SX_PART_BYTES <= K_ELEMS * 2),
                "the exchange fits in a K slot of the one-group dense kernel");
  static constexpr int NLOADW = PP ? NW / 2 : NW;  // waves sharing one tile's loads
  static_assert((KD - 1) * ((NIK + NLOADW - 1) / NLOADW + (NIV + NLOADW - 1) / NLOADW) <= 31, "vmcnt wait range");
  static_assert(CPRK >= 8 && (SPARSE || CPRV >= 8), "swizzle needs 8 chunks per row");
  static_assert(!SPARSE || (IDX_CAP % BN == 0), "index segments hold whole key blocks");
  static_assert(DQK % (16 * DS) == 0 && DV % (32 * DS) == 0, "head dims must tile");
  static_assert(!PP || (NW / 2) % DS == 0, "a query group stays inside one wave group");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
};

// ROPE > 0: the last ROPE columns of q and k come from q2 / k2 (MLA's rope
// part read in place); the other DQK - ROPE from q / k.
template <int DQK, int DV, int DS, int NW, int BN, int NBUF, bool SPARSE, bool PINGPONG, int ROPE = 0, bool XK = false,
          bool DROP = false>
__global__ void __launch_bounds__(NW * 64)
attn_fwd_dma_kernel(const KernelParams p) {
  using C = DCfg<DQK, DV, DS, NW, BN, NBUF, SPARSE, PINGPONG, XK>;
  static_assert(ROPE == 0 || (!SPARSE && DS == 1 && (DQK - ROPE) % 16 == 0 && ROPE % 16 == 0),
                "two-part rows: one wave holds the whole row, both parts whole K steps");
  static_assert(!DROP || (XK && !SPARSE && ROPE == 0 && BN == 32),
                "dropout: the one-group 512-wide kernel, one keep word per row and key block");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::LDS_BYTES];
  bf16_t* const kring = reinterpret_cast<bf16_t*>(smem);
  bf16_t* const vring = reinterpret_cast<bf16_t*>(smem + C::KRING_BYTES);
  float* const sx = reinterpret_cast<float*>(smem + C::KRING_BYTES + C::VRING_BYTES);
  int32_t* const sidx = reinterpret_cast<int32_t*>(smem + C::KRING_BYTES + C::VRING_BYTES + C::SX_BYTES);

  const int tid = threadIdx.x;
  // (the dropout instance holds the wave index in a scalar register: its key
  // loop has no vector register to spare)
  const int lane = tid & 63, wave = DROP ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int lq = lane & 31, lh = lane >> 5;
  const int qg = wave / DS, dsi = wave % DS;
  const int wgrp = C::PP ? (wave >= NW / 2 ? 1 : 0) : 0;  // wave group

  // ---------------------------------------------------------------- tile of this workgroup
  int b = 0, kvh = 0, f0 = 0, nrows = 0, t_lo = 0, t_hi = 0, sq = 0;
  // query / key counts of this workgroup's sequence, and (packed batches) the
  // sequence's first query and key token
  int Tq = p.Tq, Tk = p.Tk;
  int64_t qtok0 = 0, ktok0 = 0;
  // packed batches are compiled into the kernels up to 256-wide heads; the
  // 512-wide kernel runs at its register limit and is left without the branch
  constexpr bool kPacked = !SPARSE && DQK <= 256;
  if constexpr (SPARSE) {
    sq = blockIdx.x;
    nrows = p.H;
  } else {
    const int tile = blockIdx.x;
    if (p.fold_tm) {
      // token-major fold: tile tb of a group holds folded rows
      // [tb*BM, tb*BM + BM), row f = token f / g of head f % g
      int tb, grp;
      if (p.xcd_groups) {
        const int x = tile & 7, i = tile >> 3;
        const int per_chunk = p.xcd_chunk * p.tiles_per_group;
        const int c = i / per_chunk, r = i % per_chunk;
        tb = (p.tiles_per_group - 1) - r / p.xcd_chunk;  // longest causal tiles first
        grp = (c * p.xcd_chunk + r % p.xcd_chunk) * 8 + x;
      } else {
        tb = (p.tiles_per_group - 1) - tile / p.n_groups;
        grp = tile % p.n_groups;
      }
      b = grp / p.Hkv;
      kvh = grp % p.Hkv;
      f0 = tb * C::BM;
      if (kPacked && p.varlen) {
        // packed batch: the tiles cover the longest sequence's rows; a tile
        // past its own sequence's rows has nothing to do (every thread
        // leaves here)
        const int qs = min(max(p.cu_q[b], 0), p.total_q), qe = min(max(p.cu_q[b + 1], qs), p.total_q);
        const int ks = min(max(p.cu_k[b], 0), p.total_k), ke = min(max(p.cu_k[b + 1], ks), p.total_k);
        Tq = qe - qs;
        Tk = ke - ks;
        qtok0 = qs;
        ktok0 = ks;
        if (f0 >= p.g * Tq) return;
      }
      nrows = min(C::BM, p.g * Tq - f0);
      t_lo = f0 / p.g;
      t_hi = (f0 + nrows - 1) / p.g;
    } else if (p.aligned) {
      int tb, grp, hl;
      if (p.xcd_groups) {
        // XCD x (= tile % 8) owns groups x, x+8, ...; it takes them xcd_chunk
        // at a time, longest causal blocks first inside a chunk
        const int x = tile & 7, i = tile >> 3;
        const int per_tb = p.xcd_chunk * p.g;
        const int per_chunk = per_tb * p.tiles_per_head;
        const int c = i / per_chunk, r = i % per_chunk;
        tb = (p.tiles_per_head - 1) - r / per_tb;
        const int rest = r % per_tb;
        grp = (c * p.xcd_chunk + rest / p.g) * 8 + x;
        hl = rest % p.g;
      } else {
        const int per_tb = p.n_groups * p.g;
        tb = (p.tiles_per_head - 1) - tile / per_tb;  // longest causal blocks first
        const int rest = tile % per_tb;
        grp = rest / p.g;
        hl = rest % p.g;
      }
      b = grp / p.Hkv;
      kvh = grp % p.Hkv;
      const int t0 = tb * C::BM;
      f0 = hl * p.Tq + t0;
      nrows = min(C::BM, p.Tq - t0);
      t_lo = t0;
      t_hi = t0 + nrows - 1;
    } else {
      const int grp = tile / p.tiles_per_group;
      f0 = (tile % p.tiles_per_group) * C::BM;
      nrows = min(C::BM, p.g * p.Tq - f0);
      b = grp / p.Hkv;
      kvh = grp % p.Hkv;
      const int tf = f0 % p.Tq;
      if (nrows >= p.Tq || tf + nrows > p.Tq) {
        t_lo = 0;
        t_hi = p.Tq - 1;
      } else {
        t_lo = tf;
        t_hi = tf + nrows - 1;
      }
    }
  }
  // keys [0, kend) are needed and no row of the tile masks a key below
  // kfull; with a sliding window, none masks a key from klfull on and no row
  // sees a key before kstart. `up` = keys after a row's diagonal position it
  // may see (-1: unbounded); the window never widens the causal bound.
  int kend = Tk, kfull = Tk, kstart = 0, klfull = 0;
  const int off = Tk - Tq;
  const int up = p.causal ? 0 : p.win_right;
  if (!SPARSE && up >= 0) {
    kend = min(Tk, max(0, t_hi + off + up + 1));
    kfull = min(Tk, max(0, t_lo + off + up + 1));
  }
  if (!SPARSE && p.win_left >= 0) {
    kstart = min(Tk, max(0, t_lo + off - p.win_left));
    klfull = min(Tk, max(0, t_hi + off - p.win_left));
  }
  // this workgroup sees keys [k_lo, k_hi) only (split-KV: one range; sliding
  // window: from the block holding kstart); from here on key positions
  // (kend, kfull, klfull, the row limits, the K/V bases) are relative to k_lo
  int k_lo = 0, k_hi = Tk;
  if (!SPARSE && p.n_splits > 1) {
    k_lo = blockIdx.y * p.split_keys;
    k_hi = min(Tk, k_lo + p.split_keys);
  }
  if (!SPARSE) {
    k_lo = max(k_lo, (kstart / BN) * BN);
    kend = max(0, min(kend, k_hi) - k_lo);
    kfull = max(0, min(kfull, k_hi) - k_lo);
    klfull = max(0, klfull - k_lo);
  }

  // ---------------------------------------------------------------- the query row of this lane
  const int r = qg * 32 + lq;
  const bool row_ok = r < nrows;
  const int rr = row_ok ? r : 0;
  int row_lim, row_lo = -(1 << 30), row_h;
  int64_t q_off, o_off, l_off, q2_off = 0;
  int t_row = 0;  // the row's query token (dense)
  if constexpr (SPARSE) {
    row_h = rr;
    row_lim = Tk - 1;
    q_off = (int64_t)sq * p.q_sb + (int64_t)rr * p.q_sh;
    o_off = (int64_t)sq * p.o_sb + (int64_t)rr * p.o_sh;
    l_off = (int64_t)sq * p.H + rr;
  } else {
    const int f = f0 + rr;
    row_h = kvh * p.g + (p.fold_tm ? f % p.g : f / Tq);
    const int t = p.fold_tm ? f / p.g : f % Tq;
    row_lim = up >= 0 ? min(Tk - 1, t + off + up) : Tk - 1;
    row_lim = min(row_lim - k_lo, kend - 1);  // relative to the range
    if (p.win_left >= 0) row_lo = t + off - p.win_left - k_lo;
    q_off = (int64_t)b * p.q_sb + (int64_t)row_h * p.q_sh + (qtok0 + t) * p.q_st;
    if constexpr (ROPE > 0) q2_off = (int64_t)b * p.q2_sb + (int64_t)row_h * p.q2_sh + (qtok0 + t) * p.q2_st;
    o_off = (int64_t)b * p.o_sb + (int64_t)row_h * p.o_sh + (qtok0 + t) * p.o_st;
    t_row = t;
    l_off = kPacked && p.varlen ? (int64_t)row_h * p.total_q + qtok0 + t : ((int64_t)b * p.H + row_h) * Tq + t;
  }

  // ---------------------------------------------------------------- Q fragments (B operand of S^T)
  bf16x8 qf[C::KS];
  {
    const bf16_t* qb = reinterpret_cast<const bf16_t*>(p.q) + q_off;
    const bf16_t* qb2 = ROPE > 0 ? reinterpret_cast<const bf16_t*>(p.q2) + q2_off : nullptr;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row_ok) {
        if (ROPE > 0 && s * 16 >= DQK - ROPE)
          w = *reinterpret_cast<const u32x4*>(qb2 + (s * 16 - (DQK - ROPE)) + lh * 8);
        else
          w = *reinterpret_cast<const u32x4*>(qb + dsi * C::DQW + s * 16 + lh * 8);
      }
      qf[s] = as_bf16x8(w);
    }
    // use the fragments here so that the compiler waits for these loads before
    // the key loop, not inside it (where the wait would also drain the tile
    // loads in flight)
#pragma unroll
    for (int s = 0; s < C::KS; ++s) asm volatile("" ::"v"(qf[s]));
  }

  const bf16_t* kbase;
  const bf16_t* vbase;
  const bf16_t* k2base = nullptr;
  if constexpr (ROPE > 0)
    k2base = reinterpret_cast<const bf16_t*>(p.k2) + (int64_t)b * p.k2_sb + (int64_t)kvh * p.k2_sh +
             (ktok0 + k_lo) * p.k2_st;
  if constexpr (SPARSE) {
    kbase = reinterpret_cast<const bf16_t*>(p.k);
    vbase = kbase;
  } else {
    kbase = reinterpret_cast<const bf16_t*>(p.k) + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh + (ktok0 + k_lo) * p.k_st;
    vbase = reinterpret_cast<const bf16_t*>(p.v) + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh + (ktok0 + k_lo) * p.v_st;
  }

  // ---------------------------------------------------------------- loads of one key block
  // blk is the block index inside the current segment (sparse) or the key range (dense)
  constexpr int NLW_ = C::NLOADW;  // waves that share the loads of one tile
  constexpr int NIK_L = (C::NIK + NLW_ - 1) / NLW_, NIV_L = (C::NIV + NLW_ - 1) / NLW_;
  const int lw_ = __builtin_amdgcn_readfirstlane(wave % NLW_);
  // per-lane byte offsets of the rows and chunks a wave loads, relative to
  // the first key of the block (the swizzle is applied on the global side);
  // 32-bit because the host limits key-row strides to 2^24 elements
  auto koffg_at = [&](int m) -> uint32_t {
    const int sl = 64 * (lw_ + NLW_ * m) + lane;
    const int rw = sl / C::CPRK, c = (sl % C::CPRK) ^ swz<C::CPRK>(rw);
    return 2u * (uint32_t)(SPARSE ? c * 8 : rw * (int32_t)p.k_st + c * 8);
  };
  auto voffg_at = [&](int m) -> uint32_t {
    const int sl = 64 * (lw_ + NLW_ * m) + lane;
    const int rw = sl / C::CPRV, c = (sl % C::CPRV) ^ swz<C::CPRV>(rw);
    return 2u * (uint32_t)(rw * (int32_t)p.v_st + c * 8);
  };
  // Rows of 64 chunks (d = 512): one wave instruction loads one row, the row
  // goes into the scalar base and the per-lane part of the offset is
  // (lane ^ swizzle(row)) * 16 bytes, one XOR of lane * 16 per load. The
  // empty asm in the issue functions keeps these XORs inside the key loop
  // (hoisted, they would pin one register per load).
  constexpr bool ROWK = C::CPRK == 64, ROWV = !SPARSE && C::CPRV == 64;
  uint32_t lane16 = (uint32_t)lane << 4;
  // Rows of 8, 16 or 32 chunks: when the rows one wave's successive
  // instructions start on are a whole number of 16-row swizzle periods apart,
  // every load of the wave has the same per-lane offset and the rest is a
  // scalar step of STEPK (STEPV) rows.
  constexpr int RPIK = 64 / C::CPRK, RPIV = SPARSE ? 1 : 64 / C::CPRV;  // rows per wave instruction
  constexpr bool STRK = !ROWK && 64 % C::CPRK == 0 && (RPIK * NLW_) % 16 == 0;
  constexpr bool STRV = !SPARSE && !ROWV && 64 % C::CPRV == 0 && (RPIV * NLW_) % 16 == 0;
  constexpr int STEPK = RPIK * NLW_, STEPV = RPIV * NLW_;
  // other narrow slices keep the offsets in registers; wide ones
  // (d_qk/DS >= 256) recompute them, which is a few integer ops per load
  constexpr bool KEEPK = STRK || (C::DQW < 256 && !ROWK), KEEPV = STRV || (C::DQW < 256 && !ROWV);
  constexpr int NKG = STRK ? 1 : NIK_L, NVG = STRV ? 1 : (NIV_L > 0 ? NIV_L : 1);
  uint32_t koffg[KEEPK ? NKG : 1], voffg[KEEPV ? NVG : 1];
  if constexpr (KEEPK) {
#pragma unroll
    for (int m = 0; m < NKG; ++m) koffg[m] = koffg_at(m);
  }
  if constexpr (KEEPV && NIV_L > 0) {
#pragma unroll
    for (int m = 0; m < NVG; ++m) voffg[m] = voffg_at(m);
  }
  // The block index is the same in every lane; taking it into a scalar
  // register keeps the ring slot, the LDS address and the global base of the
  // block in scalar arithmetic.
  // (The empty asm statements below stop the per-instruction LDS addresses
  // from being hoisted out of the key loop, which would pin one scalar
  // register each.)
  const uint32_t kring_s = lds_u32(kring), vring_s = lds_u32(vring);
  auto issueK = [&](int blk_in) {
    const int blk = __builtin_amdgcn_readfirstlane(blk_in);
    uint32_t kr = kring_s + 1024u * lw_;  // this wave's first instruction slot
    asm volatile("" : "+s"(kr));
    const uint32_t Kb = kr + (uint32_t)((blk % C::NBK) * C::K_ELEMS * 2);
    const int key0 = blk * BN;
    if constexpr (ROPE > 0) {
      // two-part rows: the tile row is laid out as one DQK-wide row, chunk c
      // < NC0 comes from the first tensor and the rest from the second; the
      // lanes of one instruction cover both parts, so each carries its own
      // 64-bit address. Rows past kend are clamped onto row kend-1.
      constexpr int NC0 = (DQK - ROPE) / 8;
      const int last = kend - 1 - key0;
      const uint64_t nb = (uint64_t)(uintptr_t)(kbase + (int64_t)key0 * p.k_st);
      const uint64_t rb = (uint64_t)(uintptr_t)(k2base + (int64_t)key0 * p.k2_st);
#pragma unroll
      for (int m = 0; m < NIK_L; ++m) {
        const int j = lw_ + NLW_ * m;
        if (C::NIK % NLW_ != 0 && j >= C::NIK) break;
        const int sl = 64 * j + lane;
        const int rw = sl / C::CPRK, cp = sl % C::CPRK, c = cp ^ swz<C::CPRK>(rw);
        const int rr = min(rw, last);
        const uint64_t a = cp < NC0 ? nb + 2u * (uint32_t)(rr * (int32_t)p.k_st + c * 8)
                                    : rb + 2u * (uint32_t)(rr * (int32_t)p.k2_st + (c - NC0) * 8);
        dma16v(a, Kb + 1024u * NLW_ * m);
      }
    } else if constexpr (SPARSE) {
      // one LDS read per lane for the block's indices; each wave instruction
      // loads one pool row (64 chunks) whose index is broadcast by readlane
      static_assert(C::CPRK == 64 && BN <= 64, "one gathered row per wave instruction");
      const int myix = sidx[key0 + (lane & (BN - 1))];
      asm volatile("" : "+v"(lane16));
#pragma unroll
      for (int m = 0; m < NIK_L; ++m) {
        const int j = lw_ + NLW_ * m;
        if (C::NIK % NLW_ != 0 && j >= C::NIK) break;
        const int ix = __builtin_amdgcn_readlane(myix, j);
        const int row = (ix >= 0 && ix < p.npool) ? ix : 0;
        dma16s(uniform_ptr(kbase + (int64_t)row * p.k_st), lane16 ^ (uint32_t)(swz<64>(j) << 4), Kb + 1024u * NLW_ * m);
        static_assert(ROWK, "sparse rows are 64 chunks");
      }
    } else if constexpr (ROWK) {
      asm volatile("" : "+v"(lane16));
      const int last = kend - 1 - key0;  // rows past kend are clamped onto row kend-1
#pragma unroll
      for (int m = 0; m < NIK_L; ++m) {
        const int j = lw_ + NLW_ * m;
        if (C::NIK % NLW_ != 0 && j >= C::NIK) break;
        const int rr = min(j, last);
        dma16s(uniform_ptr(kbase + (int64_t)(key0 + rr) * p.k_st), lane16 ^ (uint32_t)(swz<64>(j) << 4),
               Kb + 1024u * NLW_ * m);
      }
    } else {
      const void* sb = uniform_ptr(kbase + (int64_t)key0 * p.k_st);
      if (key0 + BN <= kend) {
        int64_t kstep = (int64_t)STEPK * p.k_st;
        asm volatile("" : "+s"(kstep));
#pragma unroll
        for (int m = 0; m < NIK_L; ++m) {
          const int j = lw_ + NLW_ * m;
          if (C::NIK % NLW_ != 0 && j >= C::NIK) break;
          if constexpr (STRK)
            dma16s(uniform_ptr(static_cast<const bf16_t*>(sb) + m * kstep), koffg[0], Kb + 1024u * NLW_ * m);
          else
            dma16s(sb, KEEPK ? koffg[m] : koffg_at(m), Kb + 1024u * NLW_ * m);
        }
      } else {
        // last block: rows past kend are clamped onto row kend-1
#pragma unroll
        for (int m = 0; m < NIK_L; ++m) {
          const int j = lw_ + NLW_ * m;
          if (C::NIK % NLW_ != 0 && j >= C::NIK) break;
          const int sl = 64 * j + lane;
          const int rw = sl / C::CPRK, c = (sl % C::CPRK) ^ swz<C::CPRK>(rw);
          const int rr = min(rw, kend - 1 - key0);
          dma16s(sb, 2u * (uint32_t)(rr * (int32_t)p.k_st + c * 8), Kb + 1024u * NLW_ * m);
        }
      }
    }
  };
  auto issueV = [&](int blk_in) {
    if constexpr (!SPARSE) {
      const int blk = __builtin_amdgcn_readfirstlane(blk_in);
      uint32_t vr = vring_s + 1024u * lw_;
      asm volatile("" : "+s"(vr));
      const uint32_t Vb = vr + (uint32_t)((blk % NBUF) * C::V_ELEMS * 2);
      const int key0 = blk * BN;
      if constexpr (ROWV) {
        asm volatile("" : "+v"(lane16));
        const int last = kend - 1 - key0;
#pragma unroll
        for (int m = 0; m < NIV_L; ++m) {
          const int j = lw_ + NLW_ * m;
          if (C::NIV % NLW_ != 0 && j >= C::NIV) break;
          const int rr = min(j, last);
          dma16s(uniform_ptr(vbase + (int64_t)(key0 + rr) * p.v_st), lane16 ^ (uint32_t)(swz<64>(j) << 4),
                 Vb + 1024u * NLW_ * m);
        }
        return;
      }
      const void* sb = uniform_ptr(vbase + (int64_t)key0 * p.v_st);
      if (key0 + BN <= kend) {
        int64_t vstep = (int64_t)STEPV * p.v_st;
        asm volatile("" : "+s"(vstep));
#pragma unroll
        for (int m = 0; m < NIV_L; ++m) {
          const int j = lw_ + NLW_ * m;
          if (C::NIV % NLW_ != 0 && j >= C::NIV) break;
          if constexpr (STRV)
            dma16s(uniform_ptr(static_cast<const bf16_t*>(sb) + m * vstep), voffg[0], Vb + 1024u * NLW_ * m);
          else
            dma16s(sb, KEEPV ? voffg[m] : voffg_at(m), Vb + 1024u * NLW_ * m);
        }
      } else {
#pragma unroll
        for (int m = 0; m < NIV_L; ++m) {
          const int j = lw_ + NLW_ * m;
          if (C::NIV % NLW_ != 0 && j >= C::NIV) break;
          const int sl = 64 * j + lane;
          const int rw = sl / C::CPRV, c = (sl % C::CPRV) ^ swz<C::CPRV>(rw);
          const int rr = min(rw, kend - 1 - key0);
          dma16s(sb, 2u * (uint32_t)(rr * (int32_t)p.v_st + c * 8), Vb + 1024u * NLW_ * m);
        }
      }
    }
  };

  // ---------------------------------------------------------------- state
  f32x16 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // per-lane LDS offsets (elements) inside a stage; the swizzle depends on the
  // row modulo 16 only, so the mt (32 rows) and ks (16 rows) steps are
  // compile-time offsets
  constexpr int CPRVT = SPARSE ? C::CPRK : C::CPRV;  // chunks per row of the tile V is read from
  // The XOR swizzle only touches the low 4 chunk bits, so the offsets repeat
  // every 8 K steps (16 chunks) and every 4 output tiles (16 chunks) up to a
  // compile-time shift of 128 elements: keep 8 + 8 per-lane offsets.
  constexpr int NKO = C::KS < 8 ? C::KS : 8;
  constexpr int NVO = C::DT < 4 ? C::DT : 4;
  // With one wave group (wide slices, one wave per SIMD) or 128-key blocks
  // registers are scarce: for 128-aligned slices the 8 + 8 offsets are
  // rebuilt per read from a base and an XOR term (a logical K step s of a
  // row moves to chunk 2s + lh; XOR with the row swizzle sw gives
  // ((s ^ sw/2) << 1) | ((lh ^ sw) & 1) inside each 16-chunk group, and
  // likewise for the V^T quads).
  constexpr bool LEAN = (!C::PP || BN >= 128) && C::DQW % 128 == 0 && C::DVW % 128 == 0;
  int koff[LEAN ? 1 : NKO];
  int k0 = 0, kx = 0;
  if constexpr (LEAN) {
    const int sw = swz<C::CPRK>(lq);
    k0 = lq * DQK + dsi * C::DQW + (((lh ^ sw) & 1) << 3);
    kx = (sw >> 1) << 4;
  } else {
    const int sw = swz<C::CPRK>(lq);
#pragma unroll
    for (int s = 0; s < NKO; ++s)
      koff[s] = lq * DQK + (((((dsi * C::DQW + s * 16) >> 3) + lh) ^ sw) << 3);
  }
  int voff[LEAN ? 1 : NVO][2];
  int v0[2] = {0, 0}, vx[2] = {0, 0};
  if constexpr (LEAN) {
    const int vg = lane >> 4, vi = lane & 15;
    const int vrow = (vg >> 1) * 4 + (vi >> 2);
    const int r = (vg & 1) * 2 + ((vi >> 1) & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = vrow + 8 * h;
      const int sw = swz<CPRVT>(row);
      v0[h] = row * C::VLD + dsi * C::DVW + (((r ^ sw) & 3) << 3) + 4 * (vi & 1);
      vx[h] = (sw >> 2) << 5;
    }
  } else {
    const int vg = lane >> 4, vi = lane & 15;
    const int vrow = (vg >> 1) * 4 + (vi >> 2);
#pragma unroll
    for (int dt = 0; dt < NVO; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = vrow + 8 * h;
        const int col = dsi * C::DVW + dt * 32 + (vg & 1) * 16 + 4 * (vi & 3);
        voff[dt][h] = row * C::VLD + (((col >> 3) ^ swz<CPRVT>(row)) << 3) + (col & 7);
      }
  }

  f32x16 S[C::MT];
  bf16x8 pb[C::PKS];
  // dropout: the keep word of this lane's row for the current 32-key block
  // (the next block's is loaded into it once the softmax has used it); its
  // address is rebuilt per load from the row's head and token, which keeps
  // the registers of the 512-wide loop free of a 64-bit pointer
  uint32_t mw = 0u;
  auto keep_word = [&](int blk) -> uint32_t {
    int th = t_row, hh = row_h;
    asm volatile("" : "+v"(th), "+v"(hh));  // not hoisted: a 64-bit row base would stay live
    return p.keep[(int64_t)b * p.m_sb + (int64_t)hh * p.m_sh + (int64_t)th * p.m_st + (k_lo >> 5) + blk];
  };

  // S(blk) = K(blk) Q^T, partial over this wave's d_qk columns and published
  // through LDS when DS > 1
  auto doS = [&](int blk) {
    {
      const bf16_t* Kb = kring + (blk % C::NBK) * C::K_ELEMS;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[mt][i] = 0.f;
      if constexpr (LEAN) asm volatile("" : "+v"(k0), "+v"(kx));  // rebuild the offsets every step
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
          const int ko = LEAN ? k0 + ((((s % 8) << 4) ^ kx) + (s / 8) * 128) : koff[s % NKO] + (s / NKO) * 128;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + ko + mt * 32 * DQK);
          S[mt] = mfma32(a, qf[s], S[mt]);
        }
      }
      if constexpr (DS > 1 && !XK) {
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<f32x4*>(sx + (((wave * C::MT + mt) * 4 + g4) * 64 + lane) * 4) =
                f32x4{S[mt][g4 * 4], S[mt][g4 * 4 + 1], S[mt][g4 * 4 + 2], S[mt][g4 * 4 + 3]};
      }
      // keep kPrefetch operand reads in flight ahead of the MFMAs
      constexpr int PF = C::DQW >= 256 ? 3 : kPrefetch;
      constexpr int NM = C::MT * C::KS, PD = NM < PF ? NM : PF;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, PD, 0);
#pragma unroll
      for (int k = 0; k < NM - PD; ++k) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, PD, 0);
      if constexpr (DS > 1 && !XK) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 4 * C::MT, 0);
    }
  };
  // XK: the partial scores of block blk go into the K slot it was read from
  auto sx_of = [&](int blk) -> float* {
    return XK ? reinterpret_cast<float*>(kring + (blk % C::NBK) * C::K_ELEMS) : sx;
  };
  auto publishS = [&](int blk) {
    float* const d = sx_of(blk);
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(d + (((wave * C::MT + mt) * 4 + g4) * 64 + lane) * 4) =
            f32x4{S[mt][g4 * 4], S[mt][g4 * 4 + 1], S[mt][g4 * 4 + 2], S[mt][g4 * 4 + 3]};
  };

  // O += V(blk)^T P(blk), V^T fragments by transposed LDS reads; the output
  // tiles go innermost (consecutive transposed reads cover different columns,
  // measured faster for the wide slices)
  auto doPV = [&](int blk) {
    {
      const bf16_t* Vb = SPARSE ? kring + (blk % C::NBK) * C::K_ELEMS : vring + (blk % NBUF) * C::V_ELEMS;
      if constexpr (LEAN) asm volatile("" : "+v"(v0[0]), "+v"(v0[1]), "+v"(vx[0]), "+v"(vx[1]));
#pragma unroll
      for (int ks = 0; ks < C::PKS; ++ks) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const int o0 = LEAN ? v0[0] + ((((dt % 4) << 5) ^ vx[0]) + (dt / 4) * 128) : voff[dt % NVO][0] + (dt / NVO) * 128;
          const int o1 = LEAN ? v0[1] + ((((dt % 4) << 5) ^ vx[1]) + (dt / 4) * 128) : voff[dt % NVO][1] + (dt / NVO) * 128;
          const bf16_t* p0 = Vb + o0 + ks * 16 * C::VLD;
          const bf16_t* p1 = Vb + o1 + ks * 16 * C::VLD;
          const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
          const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
          const u32x4 w = {(uint32_t)(uint16_t)t0[0] | ((uint32_t)(uint16_t)t0[1] << 16),
                           (uint32_t)(uint16_t)t0[2] | ((uint32_t)(uint16_t)t0[3] << 16),
                           (uint32_t)(uint16_t)t1[0] | ((uint32_t)(uint16_t)t1[1] << 16),
                           (uint32_t)(uint16_t)t1[2] | ((uint32_t)(uint16_t)t1[3] << 16)};
          acc[dt] = mfma32(as_bf16x8(w), pb[ks], acc[dt]);
        }
      }
      // two transposed reads per MFMA; keep kPrefetch MFMAs' operands in flight
      constexpr int PF = C::DVW >= 256 ? 2 : kPrefetch;
      constexpr int NM = C::DT * C::PKS, PD = NM < PF ? NM : PF;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * PD, 0);
#pragma unroll
      for (int k = 0; k < NM - PD; ++k) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, PD, 0);
    }
  };

  // VALU half of a key step: full scores, masks, online softmax -> P(blk)
  auto phase2 = [&](int blk) {
    const int key0 = blk * BN;
    if constexpr (DS > 1) {
      const float* const sxb = sx_of(blk);
#pragma unroll
      for (int o = 1; o < DS; ++o) {
        const int w2 = qg * DS + (dsi + o) % DS;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(sxb + (((w2 * C::MT + mt) * 4 + g4) * 64 + lane) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[mt][g4 * 4 + e] += v[e];
          }
      }
    }
    if constexpr (SPARSE) {
      // lane k tests key k of the block; the ballot has a set bit per key
      // whose index is out of range (padding of a short list, or invalid)
      static_assert(BN <= 64, "one key per lane");
      const int ixl = sidx[key0 + (lane & (BN - 1))];
      uint64_t bad = __ballot(ixl < 0 || ixl >= p.npool);
      if constexpr (BN < 64) bad &= (uint64_t(1) << BN) - 1;
      if (bad != 0) {
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if ((bad >> (mt * 32 + (i >> 2) * 8 + lh * 4 + (i & 3))) & 1) S[mt][i] = -INFINITY;
      }
    } else {
      if (key0 + BN > kfull) {
        const int lim = row_lim - key0 - lh * 4;  // mask keys whose in-block offset exceeds lim
        // branch-free select from the sign of lim - offset (v_sub, v_ashr,
        // v_bfi); compares against the 16 * MT constants would each hold a
        // 64-bit lane mask in scalar registers
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int over = (lim - (mt * 32 + (i >> 2) * 8 + (i & 3))) >> 31;  // all ones past the limit
            S[mt][i] = __int_as_float((__float_as_int(S[mt][i]) & ~over) | (int)(0xff800000u & (uint32_t)over));
          }
      }
      if (key0 < klfull) {
        // sliding window: mask keys before the row's window (offset below lo)
        const int lo = row_lo - key0 - lh * 4;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int under = ((mt * 32 + (i >> 2) * 8 + (i & 3)) - lo) >> 31;  // all ones before the window
            S[mt][i] = __int_as_float((__float_as_int(S[mt][i]) & ~under) | (int)(0xff800000u & (uint32_t)under));
          }
      }
    }
    // four partial maxima and sums keep the dependency chains short
    float mx4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx4[i & 3] = fmaxf(mx4[i & 3], S[mt][i]);
    const float mx = halves_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])));
    const float mnew = fmaxf(m_run, mx);
    const bool grow = (mnew - m_run) * p.c > kRescaleLog2;  // false when both are -inf
    if (__any(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - mnew) * p.c) : 1.f;
      if (grow) m_run = mnew;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * p.c;
    float rs4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(fmaf(S[mt][i], p.c, -mc));
        rs4[i & 3] += e;
        // dropout: the denominator takes every probability, the product with
        // V only the kept ones (key mt*32 + lh*4 + 8*(i/4) + i%4 of the block)
        if constexpr (DROP) S[mt][i] = ((mw >> (mt * 32 + lh * 4 + 8 * (i >> 2) + (i & 3))) & 1u) ? e : 0.f;
        else S[mt][i] = e;
      }
    l_run += (rs4[0] + rs4[1]) + (rs4[2] + rs4[3]);
#pragma unroll
    for (int ks = 0; ks < C::PKS; ++ks) {
      const int mt = ks >> 1, base = (ks & 1) * 8;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(S[mt][base + 2 * e], S[mt][base + 2 * e + 1]);
      pb[ks] = as_bf16x8(w);
    }
  };

  // ---------------------------------------------------------------- key loop
  // Key step i spans barriers B(2i) .. B(2i+2). With two groups, group 0 runs
  // its MFMA half (S(i), PV(i-1)) then its softmax half (phase2(i)); group 1
  // runs phase2(i-1) then S(i), PV(i-1), so on every SIMD one wave multiplies
  // while the other does the softmax; step nb only drains the last PV
  // product. With one group a step is S(i), [exchange], phase2(i), PV(i).
  // with two groups each group's waves load one tile kind (K: group 0, V: group 1)
  const int myK = C::NIK / NLW_ + (lw_ < C::NIK % NLW_ ? 1 : 0);
  const int myV = C::NIV / NLW_ + (lw_ < C::NIV % NLW_ ? 1 : 0);
  const int nseg = SPARSE ? (p.Tk + C::IDX_CAP - 1) / max(C::IDX_CAP, 1) : 1;
  for (int sg = 0; sg < nseg; ++sg) {
    int nb;
    if constexpr (SPARSE) {
      const int seg0 = sg * C::IDX_CAP;
      const int segn = min(C::IDX_CAP, p.Tk - seg0);
      nb = (segn + BN - 1) / BN;
      if (sg > 0) lds_barrier();  // everyone is done with the previous segment's indices and tiles
      const int32_t* irow = p.idx + (int64_t)sq * p.idx_ss + seg0;
      for (int e = tid; e < nb * BN; e += C::NT) sidx[e] = (e < segn) ? irow[e] : -1;
      lds_barrier();
    } else {
      nb = (kend + BN - 1) / BN;
    }
    // Loads of key step i: K block i+KD and V block i+VD. With two groups the
    // V block is loaded by group 1 right after B(2i), at the start of its
    // softmax half, and the K block by group 0 in the same half step, between
    // the S and PV products of its MFMA half (measured 1% faster than at the
    // start of its softmax half, which the VALU work makes the longer half);
    // with one group both are issued right after the S product of step i,
    // while its MFMAs drain.
    auto issue_k = [&](int i) {
      const int kj = i + C::KD;
      if (kj >= 0 && kj < nb) issueK(kj);
    };
    auto issue_v = [&](int i) {
      const int vj = i + C::VD;
      if (!SPARSE && vj >= 0 && vj < nb) issueV(vj);
    };
    // loads of step i that this wave issued (it only counts its own)
    auto step_loads = [&](int i) {
      const int kj = i + C::KD, vj = i + C::VD;
      const bool doesK = !C::PP || wgrp == 0, doesV = !C::PP || wgrp == 1 || SPARSE;
      return ((doesK && kj >= 0 && kj < nb) ? myK : 0) + ((doesV && !SPARSE && vj >= 0 && vj < nb) ? myV : 0);
    };
    auto issue_step = [&](int i) {
      issue_k(i);
      issue_v(i);
    };
    if constexpr (DROP) {
      if (nb > 0) mw = keep_word(0);
    }
    for (int i = -C::KD; i < 0; ++i) {
      if constexpr (XK) {
        // issue order K 0, V 0, K 1: at step j only K block j+1 may stay in flight
        issue_v(i);
        issue_k(i);
      } else {
        if (!C::PP || wgrp == 0) issue_k(i);
        if (!C::PP || wgrp == 1) issue_v(i);
      }
    }
    // wait until K block i and V block i-1 (two groups) or V block i (one
    // group) have landed: they were issued at B(2(i-KD)), later loads may
    // stay in flight
    auto wait_step = [&](int i) {
      int allow = 0;
#pragma unroll
      for (int g = 1; g < C::KD; ++g) allow += step_loads(i - g);
      wait_vmcnt_dyn(allow);
    };
    if constexpr (C::PP) {
      // half-step t: barrier B(t); one call site per phase keeps register
      // allocation to a single path
      for (int t = 0; t <= 2 * nb + 1; ++t) {
        // Only even half steps synchronise: every load's landing (waited
        // just before) and every ring-slot reuse is separated from its
        // readers by one of them, so the groups need not meet in between.
        if ((t & 1) == 0) {
          wait_step(t >> 1);
          lds_barrier();
        }
        const int u = t - wgrp;
        if (u < 0) {
          issue_v(t >> 1);  // group 1, half-step 0
          continue;
        }
        const int j = u >> 1;
        if ((u & 1) == 0) {
          // MFMA half: S(j) and the PV product of block j-1; group 0's K
          // loads of step t/2 go out between the two, while the S products
          // drain
          if (j < nb) doS(j);
          // keep the V reads below the S product (register pressure)
          __builtin_amdgcn_sched_barrier(0);
          if (wgrp == 0) issue_k(t >> 1);
          if (j >= 1) doPV(j - 1);
        } else {
          // softmax half; group 1's V loads of step t/2 go first
          if (wgrp == 1) issue_v(t >> 1);
          if (j < nb) phase2(j);
        }
      }
    } else if constexpr (XK) {
      // step j: V block j+1 and K block j+2 are issued (in that order) into
      // the slots step j-1 finished with, before the S product; the partial
      // scores are exchanged in K block j's slot between two barriers. With
      // dropout every step drains the loads (K block j+1 included): the keep
      // word of block j+1 is an ordinary load, issued once the softmax of
      // block j has used the register, and the compiler's wait for it then
      // falls after the drain
      for (int j = 0; j < nb; ++j) {
        if constexpr (DROP)
          wait_vmcnt_dyn(0);
        else
          wait_vmcnt_dyn(j + 1 < nb ? myK : 0);  // K block j and V block j have landed
        lds_barrier();
        if constexpr (DROP) asm volatile("" ::"v"(mw));  // the compiler's wait for the word lands here
        issue_v(j);
        issue_k(j);
        doS(j);
        lds_barrier();  // every wave has read K block j
        publishS(j);
        lds_barrier();
        phase2(j);
        if constexpr (DROP) {
          if (j + 1 < nb) mw = keep_word(j + 1);
        }
        doPV(j);
      }
    } else {
      for (int j = 0; j < nb; ++j) {
        wait_step(j);
        lds_barrier();
        doS(j);
        // the loads go out while the queued S products execute
        issue_step(j);
        if constexpr (DS > 1) lds_barrier();  // publishes the partial scores
        phase2(j);
        doPV(j);
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
  const float lt = halves_sum(l_run);
  const float ms = (m_run == -INFINITY) ? -INFINITY : m_run * p.scale;
  if (!SPARSE && !DROP && p.n_splits > 1) {  // (the host never splits a dropout launch)
    // split-KV partial: O over this key range normalised by the range's own
    // denominator (fp32), lse of the range without the sink
    if (row_ok) {
      const float pinv = lt > 0.f ? 1.f / lt : 0.f;
      const int64_t prow = (int64_t)blockIdx.y * ((int64_t)p.B * p.H * p.Tq) + l_off;
      float* po = p.part_o + prow * DV;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = dsi * C::DVW + dt * 32 + g4 * 8 + lh * 4;
          *reinterpret_cast<f32x4*>(po + d) = f32x4{acc[dt][g4 * 4] * pinv, acc[dt][g4 * 4 + 1] * pinv,
                                                    acc[dt][g4 * 4 + 2] * pinv, acc[dt][g4 * 4 + 3] * pinv};
        }
      if (lh == 0 && dsi == 0) p.part_lse[prow] = lt > 0.f ? ms + __builtin_amdgcn_logf(lt) * kLn2 : -INFINITY;
    }
    return;
  }
  float inv, lse;
  if (p.sinks != nullptr) {
    const float sk = p.sinks[row_h];
    const float M = fmaxf(ms, sk);
    if (M == -INFINITY) {
      inv = 0.f;
      lse = -INFINITY;
    } else {
      const float fac = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((ms - M) * kLog2e);
      const float es = (sk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((sk - M) * kLog2e);
      const float den = lt * fac + es;
      inv = den > 0.f ? fac / den : 0.f;
      lse = den > 0.f ? M + __builtin_amdgcn_logf(den) * kLn2 : -INFINITY;
    }
  } else {
    inv = lt > 0.f ? 1.f / lt : 0.f;
    lse = lt > 0.f ? ms + __builtin_amdgcn_logf(lt) * kLn2 : -INFINITY;
  }
  if constexpr (DROP) {
    inv *= p.inv_keep;  // the kept probabilities are scaled by 1 / (1 - p)
    // rebuilt here rather than kept live through the key loop (registers)
    o_off = (int64_t)b * p.o_sb + (int64_t)row_h * p.o_sh + (int64_t)t_row * p.o_st;
    l_off = ((int64_t)b * p.H + row_h) * Tq + t_row;
  }
  if (row_ok) {
    bf16_t* ob = reinterpret_cast<bf16_t*>(p.out) + o_off;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dsi * C::DVW + dt * 32 + g4 * 8 + lh * 4;
        *reinterpret_cast<u32x2*>(ob + d) =
            u32x2{pack_bf16x2(acc[dt][g4 * 4] * inv, acc[dt][g4 * 4 + 1] * inv),
                  pack_bf16x2(acc[dt][g4 * 4 + 2] * inv, acc[dt][g4 * 4 + 3] * inv)};
      }
    // both lane halves of a row hold the same lse; the dropout instance lets
    // both store it (the lane half is not kept live through its key loop)
    if ((DROP || lh == 0) && dsi == 0) p.lse[l_off] = lse;
  }
}

template <int DQK, int DV, int DS, int NW, int BN, int NBUF, bool PINGPONG, bool SPARSE, int ROPE = 0, bool XK = false,
          bool DROP = false>
int occupancy_dma() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n,
          reinterpret_cast<const void*>(&attn_fwd_dma_kernel<DQK, DV, DS, NW, BN, NBUF, SPARSE, PINGPONG, ROPE, XK, DROP>),
          NW * 64, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

template <int DQK, int DV, int DS, int NW, int BN, int NBUF, bool PINGPONG, bool SPARSE, int ROPE = 0, bool XK = false,
          bool DROP = false>
int launch_dma(const KernelParams& p, void* stream) {
  hipLaunchKernelGGL((attn_fwd_dma_kernel<DQK, DV, DS, NW, BN, NBUF, SPARSE, PINGPONG, ROPE, XK, DROP>),
                     dim3(p.n_tiles, p.n_splits > 1 ? p.n_splits : 1), dim3(NW * 64), 0,
                     reinterpret_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

// ===========================================================================
// Merge of split-KV partials: one wave per query row. Each key range i left
// (O_i normalised by its own denominator, lse_i without the sink); then
// lse = log(sum_i exp(lse_i) [+ exp(sink)]) and O = sum_i exp(lse_i - lse) O_i
// (the output merge of TransformerEngine's context-parallel forward,
// "Flowchart", done across workgroups of one device). Memory bound: it reads
// n_splits * d_v floats per row once.
// ===========================================================================
__global__ void __launch_bounds__(256) merge_splits_kernel(const MergeParams m) {
  const int lane = threadIdx.x & 63;
  const int64_t R = (int64_t)m.B * m.H * m.Tq;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  const int t = (int)(row % m.Tq);
  const int h = (int)((row / m.Tq) % m.H);
  const int b = (int)(row / ((int64_t)m.Tq * m.H));
  const int n = m.n_splits, nc = m.d_v / 4;
  const float sk = m.sinks != nullptr ? m.sinks[h] : -INFINITY;
  const int64_t obase = (int64_t)b * m.o_sb + (int64_t)h * m.o_sh + (int64_t)t * m.o_st;
  // The wave's lanes split into G groups of C lanes: lane (c, s) takes 4-float
  // chunk c of ranges s, s + G, s + 2G, ..., U of them per batch, loading each
  // range's partial and its lse together (one memory round trip per batch).
  // C is the smallest of 16, 32, 64 that holds the row's d_v / 4 chunks; wider
  // rows take several passes. Sums run relative to the running maximum M of
  // the lse_i seen so far; the groups add up across lanes at the end.
  constexpr int U = 16;
  const int C = nc <= 16 ? 16 : (nc <= 32 ? 32 : 64), G = 64 / C;
  const int s = lane / C;
  for (int c0 = 0; c0 < nc; c0 += C) {
    const int c = c0 + lane % C;
    const bool on = c < nc;
    const float* po = m.part_o + row * m.d_v + 4 * (on ? c : nc - 1);
    float M = -INFINITY, den = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < n; i0 += U * G) {
      float li[U];
      f32x4 oi[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + s + u * G;
        if (i < n) {
          li[u] = m.part_lse[i * R + row];
          oi[u] = *reinterpret_cast<const f32x4*>(po + i * R * m.d_v);
        } else {
          li[u] = -INFINITY;
          oi[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      float bm = li[0];
#pragma unroll
      for (int u = 1; u < U; ++u) bm = fmaxf(bm, li[u]);
      for (int x = C; x < 64; x <<= 1) bm = fmaxf(bm, __shfl_xor(bm, x, 64));
      const float Mn = fmaxf(M, bm);
      if (Mn == -INFINITY) continue;  // no range with keys yet
      const float a = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
      den *= a;
      o *= a;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // an empty range (lse_i = -inf) adds nothing, whatever its partial holds
        const bool empty = li[u] == -INFINITY;
        const float w = empty ? 0.f : __builtin_amdgcn_exp2f((li[u] - Mn) * kLog2e);
        den += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] += empty ? 0.f : w * oi[u][e];
      }
      M = Mn;
    }
    for (int x = C; x < 64; x <<= 1) {
      den += __shfl_xor(den, x, 64);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += __shfl_xor(o[e], x, 64);
    }
    // the sink joins the denominator
    const float Mx = fmaxf(M, sk);
    float lse = -INFINITY, f = 0.f;
    if (Mx != -INFINITY) {
      const float fa = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((M - Mx) * kLog2e);
      const float dt = den * fa + ((sk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((sk - Mx) * kLog2e));
      if (dt > 0.f) {
        lse = Mx + __builtin_amdgcn_logf(dt) * kLn2;
        f = fa / dt;
      }
    }
    o *= f;
    if (on && s == 0) {
      if (m.f32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(m.out) + obase + 4 * c) = o;
      } else {
        *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(m.out) + obase + 4 * c) =
            u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      }
    }
    if (c0 == 0 && lane == 0) m.lse[row] = lse;
  }
}

#define DMA_ENTRY_ROPE(NAME, DQK, DV, ROPE, DS, NW, BN, NBUF, PP)                                                  \
  KernelConfig {                                                                                                 \
    NAME, 0, DQK, DV, false, DCfg<DQK, DV, DS, NW, BN, NBUF, false, PP>::BM, BN, NW,                               \
        DCfg<DQK, DV, DS, NW, BN, NBUF, false, PP>::LDS_BYTES, &launch_dma<DQK, DV, DS, NW, BN, NBUF, PP, false, ROPE>, \
        &occupancy_dma<DQK, DV, DS, NW, BN, NBUF, PP, false, ROPE>, ROPE                                          \
  }

#define DMA_ENTRY_XK(NAME, DQK, DV, DS, NW, BN, NBUF, PP, XK)                                                    \
  KernelConfig {                                                                                                 \
    NAME, 0, DQK, DV, false, DCfg<DQK, DV, DS, NW, BN, NBUF, false, PP, XK>::BM, BN, NW,                          \
        DCfg<DQK, DV, DS, NW, BN, NBUF, false, PP, XK>::LDS_BYTES, &launch_dma<DQK, DV, DS, NW, BN, NBUF, PP, false, 0, XK>, \
        &occupancy_dma<DQK, DV, DS, NW, BN, NBUF, PP, false, 0, XK>                                              \
  }

#define DMA_ENTRY_XK_DROP(NAME, DQK, DV, DS, NW, BN, NBUF, PP, XK)                                               \
  KernelConfig {                                                                                                 \
    NAME, 0, DQK, DV, false, DCfg<DQK, DV, DS, NW, BN, NBUF, false, PP, XK>::BM, BN, NW,                          \
        DCfg<DQK, DV, DS, NW, BN, NBUF, false, PP, XK>::LDS_BYTES,                                               \
        &launch_dma<DQK, DV, DS, NW, BN, NBUF, PP, false, 0, XK, true>,                                          \
        &occupancy_dma<DQK, DV, DS, NW, BN, NBUF, PP, false, 0, XK, true>, 0, 1                                  \
  }

#define DMA_ENTRY(NAME, DQK, DV, DS, NW, BN, NBUF, PP, SPARSE)                                                   \
  KernelConfig {                                                                                                 \
    NAME, 0, DQK, DV, SPARSE, DCfg<DQK, DV, DS, NW, BN, NBUF, SPARSE, PP>::BM, BN, NW,                           \
        DCfg<DQK, DV, DS, NW, BN, NBUF, SPARSE, PP>::LDS_BYTES, &launch_dma<DQK, DV, DS, NW, BN, NBUF, PP, SPARSE>, \
        &occupancy_dma<DQK, DV, DS, NW, BN, NBUF, PP, SPARSE>                                                    \
  }

template <int DQK, int DV, int QT, int DS, int NW, int BN, bool F32, bool SPARSE>
int occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&attn_fwd_kernel<DQK, DV, QT, DS, NW, BN, F32, SPARSE>), NW * 64, 0) !=
      hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

template <int DQK, int DV, int QT, int DS, int NW, int BN, bool F32, bool SPARSE>
int launch(const KernelParams& p, void* stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<DQK, DV, QT, DS, NW, BN, F32, SPARSE>), dim3(p.n_tiles), dim3(NW * 64), 0,
                     reinterpret_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

#define CFG_ENTRY(NAME, DT, DQK, DV, QT, DS, NW, BN, F32, SPARSE)                                          \
  KernelConfig {                                                                                          \
    NAME, DT, DQK, DV, SPARSE, Cfg<DQK, DV, QT, DS, NW, BN, F32, SPARSE>::BM, BN, NW,                    \
        Cfg<DQK, DV, QT, DS, NW, BN, F32, SPARSE>::LDS_BYTES, &launch<DQK, DV, QT, DS, NW, BN, F32, SPARSE>, \
        &occupancy<DQK, DV, QT, DS, NW, BN, F32, SPARSE>                                                   \
  }

// (DS, waves, BN, LDS ring slots, two wave groups) per head-dim configuration;
// DMA_ENTRY_X expands them first
#define DMA_ENTRY_X(...) DMA_ENTRY(__VA_ARGS__)
#define DMA_ENTRY_ROPE_X(...) DMA_ENTRY_ROPE(__VA_ARGS__)
#define DMA_ENTRY_XK_X(...) DMA_ENTRY_XK(__VA_ARGS__)
#define DMA_ENTRY_XK_DROP_X(...) DMA_ENTRY_XK_DROP(__VA_ARGS__)
#ifndef ATTN_CFG_D64
#define ATTN_CFG_D64 1, 8, 64, 3, true
#endif
#ifndef ATTN_CFG_D128
#define ATTN_CFG_D128 1, 8, 128, 2, true
#endif
#ifndef ATTN_CFG_D192
#define ATTN_CFG_D192 1, 8, 64, 3, true
#endif
#ifndef ATTN_CFG_D256
#define ATTN_CFG_D256 2, 4, 32, 3, false
#endif
#ifndef ATTN_CFG_D512
#define ATTN_CFG_D512 2, 8, 32, 2, false
#endif
#ifndef ATTN_D512_XK
#define ATTN_D512_XK true
#endif
#ifndef ATTN_CFG_SPARSE
#define ATTN_CFG_SPARSE 4, 8, 32, 3, false
#endif

const KernelConfig kTable[] = {
    DMA_ENTRY_X("dense_bf16_d64", 64, 64, ATTN_CFG_D64, false),
    DMA_ENTRY_X("dense_bf16_d128", 128, 128, ATTN_CFG_D128, false),
    DMA_ENTRY_X("dense_bf16_d192_v128", 192, 128, ATTN_CFG_D192, false),
    DMA_ENTRY_ROPE_X("dense_bf16_d192_v128_rope64", 192, 128, 64, ATTN_CFG_D192),
    DMA_ENTRY_X("dense_bf16_d256", 256, 256, ATTN_CFG_D256, false),
    DMA_ENTRY_XK_X("dense_bf16_d512", 512, 512, ATTN_CFG_D512, ATTN_D512_XK),
    DMA_ENTRY_XK_DROP_X("dense_bf16_d512_dropout", 512, 512, ATTN_CFG_D512, ATTN_D512_XK),
    CFG_ENTRY("dense_f32split_d64", 1, 64, 64, 1, 1, 4, 32, true, false),
    CFG_ENTRY("dense_f32split_d128", 1, 128, 128, 1, 1, 4, 32, true, false),
    DMA_ENTRY_X("sparse_bf16_d512", 512, 512, ATTN_CFG_SPARSE, true),
    DMA_ENTRY_X("sparse_bf16_d512_v384", 512, 384, ATTN_CFG_SPARSE, true),
    DMA_ENTRY_X("sparse_bf16_d512_v256", 512, 256, ATTN_CFG_SPARSE, true),
    DMA_ENTRY_X("sparse_bf16_d512_v128", 512, 128, ATTN_CFG_SPARSE, true),
};

}  // namespace

const KernelConfig* kernel_table(int* n) {
  *n = (int)(sizeof(kTable) / sizeof(kTable[0]));
  return kTable;
}

int launch_merge(const MergeParams& m, void* stream) {
  const int64_t rows = (int64_t)m.B * m.H * m.Tq;
  hipLaunchKernelGGL(merge_splits_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), m);
  return (int)hipGetLastError();
}

}  // namespace attn
