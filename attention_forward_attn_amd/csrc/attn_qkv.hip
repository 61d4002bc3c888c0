// Decode attention over a quantized K/V cache for AMD CDNA4 (gfx950).
//
// K and V are stored in llama.cpp's q8_0 or q4_0 block formats (blocks of 32
// values along the head dimension: an fp16 scale, then 32 int8 codes or 16
// bytes of 4-bit codes). The llama.cpp page ("Pins #303") describes the point
// of the in-kernel path: the attention kernel dequantizes the K/V tiles it
// loads, instead of converting the whole cache to f16 on every step. Here each
// 32-key tile goes from global memory into LDS as raw bytes (coalesced dword
// loads), is decoded by the wave into f16 tiles in LDS, and feeds f16 MFMAs:
//
//   S^T = K Q^T      v_mfma_f32_32x32x16_f16, the lane owns one query row
//   online softmax   as in the bf16 forward (base-2, lane-local row state)
//   O^T += V^T P^T   V^T fragments by transposed LDS reads of the f16 tile
//
// f16 keeps the decoded values to 11 significant bits (a q8_0 value d*q needs
// up to 18) where bf16 would keep 8; q is converted from bf16 exactly.
//
// One wave per workgroup: a workgroup owns up to 32 folded query rows (GQA:
// the g heads x Tq tokens of one kv head, e.g. 4 heads x 4 tokens of a
// multi-sequence decode step) and one range of keys (grid y), writing the
// range's partial result for the split-KV merge; with one range it writes
// out and lse directly.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_params.h"

namespace attn {
namespace {

typedef _Float16 f16_t;
typedef __bf16 bf16_t;
typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef f16_t f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kFmtQ8 = 8, kFmtQ4 = 2;  // the ggml type numbers of q8_0 and q4_0

__device__ __forceinline__ f32x16 mfma16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// two floats -> two f16 (round to nearest even) in one 32-bit word
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  const uint32_t a = __builtin_bit_cast(uint16_t, (f16_t)lo), b = __builtin_bit_cast(uint16_t, (f16_t)hi);
  return a | (b << 16);
}

// two floats -> two bf16 (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// The raw tiles are written as 32-bit words and read as 16-bit halves, the
// f16 tiles written as 128-bit chunks and read as MFMA operands: a compiler
// barrier keeps these differently typed LDS accesses in program order (the
// wave's LDS operations then complete in order).
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_u32(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ptr;
}

__device__ __forceinline__ const void* uniform_ptr(const void* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// 4 bytes per lane from global memory straight into LDS at m0 + 4 * lane
// (wave-uniform base in scalar registers, per-lane 32-bit byte offset); the
// compiler does not see these loads, so their waits are explicit
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// 16-byte chunk swizzle of a tile row with CPR chunks (64 LDS banks), as in
// the bf16 kernels: 16 consecutive rows put one logical chunk in distinct bank
// groups, aligned 4-row groups put a 4-chunk group in distinct groups.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  static_assert(CPR % 16 == 0, "rows of whole 256-byte groups");
  return ((r & 3) << 2) | ((r >> 2) & 3);
}

template <int CPR>
__device__ __forceinline__ int chunk_at(int r, int c) {
  return r * (CPR * 8) + ((c ^ swz<CPR>(r)) << 3);
}

// A operand rows: lane row `row`, columns 16s + 8lh .. +7
template <int CPR>
__device__ __forceinline__ f16x8 row_frag(const f16_t* tile, int row, int s, int lh) {
  return *reinterpret_cast<const f16x8*>(tile + chunk_at<CPR>(row, 2 * s + lh));
}

// A operand X^T (32 columns by 16 rows r0..r0+15) by two transposed reads; the
// rows arrive in the order the B operand built from a 32x32 accumulator takes
// them (elements 8ks .. 8ks+7)
template <int CPR>
__device__ __forceinline__ f16x8 tr_frag(const f16_t* tile, int r0, int c0, int lane) {
  const int vg = lane >> 4, vi = lane & 15;
  const int vrow = (vg >> 1) * 4 + (vi >> 2);
  const int col = c0 + (vg & 1) * 16 + 4 * (vi & 3);
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = r0 + vrow + 8 * h;
    const f16_t* ptr = tile + row * (CPR * 8) + (((col >> 3) ^ swz<CPR>(row)) << 3) + (col & 7);
    const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)ptr);
    w[2 * h] = (uint32_t)(uint16_t)t[0] | ((uint32_t)(uint16_t)t[1] << 16);
    w[2 * h + 1] = (uint32_t)(uint16_t)t[2] | ((uint32_t)(uint16_t)t[3] << 16);
  }
  return __builtin_bit_cast(f16x8, u32x4{w[0], w[1], w[2], w[3]});
}

// Decode 8 consecutive values (elements w0..w0+7 of one block, w0 a multiple
// of 8) of the raw block at byte `bb` of the LDS byte array `raw` into 4 words
// of packed f16.
//
// Packed f16 arithmetic: a byte b (0..255) placed under the exponent bits
// 0x64 is the f16 number 1024 + b exactly, so codes become f16 with one
// byte permute and one OR per pair, the offset (1024 + 128 for int8 codes
// stored with their sign bit flipped, 1024 + 8 for nibbles) goes with one
// packed subtract, and the scale with one packed multiply (d * code rounded
// once to f16, as a single f32 product rounded to f16 would be).
typedef f16_t f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t scale_pair(uint32_t four_bytes_lo_hi, uint32_t sel, f16x2 offset, f16x2 d2) {
  const uint32_t bits = __builtin_amdgcn_perm(0u, four_bytes_lo_hi, sel) | 0x64006400u;
  const f16x2 v = (__builtin_bit_cast(f16x2, bits) - offset) * d2;
  return __builtin_bit_cast(uint32_t, v);
}

template <int FMT>
__device__ __forceinline__ u32x4 decode8(const unsigned char* raw, int bb, int w0) {
  const f16_t d = __builtin_bit_cast(f16_t, *reinterpret_cast<const uint16_t*>(raw + bb));
  const f16x2 d2 = {d, d};
  // the 8 code bytes (q8_0) or the 8 bytes holding the nibbles (q4_0), read as
  // 2-byte halves (blocks are 2-byte aligned)
  const uint16_t* cp = reinterpret_cast<const uint16_t*>(raw + bb + 2 + (FMT == kFmtQ8 ? w0 : (w0 & 15)));
  uint32_t lo = (uint32_t)cp[0] | ((uint32_t)cp[1] << 16), hi = (uint32_t)cp[2] | ((uint32_t)cp[3] << 16);
  f16x2 off;
  if constexpr (FMT == kFmtQ8) {
    lo ^= 0x80808080u;  // int8 q -> q + 128
    hi ^= 0x80808080u;
    off = f16x2{(f16_t)1152.f, (f16_t)1152.f};
  } else {
    // element e < 16: low nibble of byte e; element e >= 16: high nibble of byte e - 16
    const int sh = w0 >= 16 ? 4 : 0;
    lo = (lo >> sh) & 0x0f0f0f0fu;
    hi = (hi >> sh) & 0x0f0f0f0fu;
    off = f16x2{(f16_t)1032.f, (f16_t)1032.f};
  }
  // byte k of the result pair: selector 0..3 picks byte k of the second
  // operand, 0x0c gives 0
  return u32x4{scale_pair(lo, 0x0c010c00u, off, d2), scale_pair(lo, 0x0c030c02u, off, d2),
               scale_pair(hi, 0x0c010c00u, off, d2), scale_pair(hi, 0x0c030c02u, off, d2)};
}

template <int FMT, int D>
__global__ void __launch_bounds__(64) qkv_decode_kernel(const QkvParams p) {
  constexpr int BN = 32;                          // keys per tile
  constexpr int BB = FMT == kFmtQ8 ? 34 : 18;     // bytes per 32-value block
  constexpr int RB = D / 32 * BB;                 // bytes per cache row
  constexpr int RAW_DW = BN * RB / 4;             // dwords of one raw tile
  constexpr int RAW_PL = RAW_DW / 64;             // per lane
  constexpr int CPR = D / 8, KS = D / 16, DT = D / 32;
  constexpr int CH_PL = BN * CPR / 64;            // decoded 8-value chunks per lane per tile
  static_assert(RB % 4 == 0 && RAW_DW % 64 == 0 && (BN * CPR) % 64 == 0, "tile shapes");
  // raw tiles, two stages each (the next tile lands while this one is decoded)
  __shared__ __attribute__((aligned(16))) uint32_t rawk[2][RAW_DW];
  __shared__ __attribute__((aligned(16))) uint32_t rawv[2][RAW_DW];
  __shared__ __attribute__((aligned(16))) f16_t kt[BN * D];
  __shared__ __attribute__((aligned(16))) f16_t vt[BN * D];

  const int lane = threadIdx.x, lq = lane & 31, lh = lane >> 5;
  const int grp = blockIdx.x / p.n_rt, rt = blockIdx.x % p.n_rt;
  const int b = grp / p.Hkv, kvh = grp % p.Hkv;
  const int rows = p.g * p.Tq;
  const int f0 = rt * 32, f = f0 + lq;
  const bool valid = f < rows;
  const int fc = valid ? f : rows - 1;
  const int h = kvh * p.g + fc / p.Tq, t = fc % p.Tq;
  const int off = p.Tk - p.Tq;

  // keys the tile's rows can see, then this workgroup's key range
  int kend = p.Tk;
  if (p.causal) {
    const int f_last = min(f0 + 32, rows) - 1;
    const int t_hi = (f_last / p.Tq != f0 / p.Tq) ? p.Tq - 1 : f_last % p.Tq;
    kend = min(p.Tk, max(0, t_hi + off + 1));
  }
  int k_lo = 0, k_hi = p.Tk;
  if (p.n_splits > 1) {
    k_lo = blockIdx.y * p.split_keys;
    k_hi = min(p.Tk, k_lo + p.split_keys);
  }
  kend = max(0, min(kend, k_hi) - k_lo);
  int row_lim = valid ? (p.causal ? min(p.Tk - 1, t + off) : p.Tk - 1) - k_lo : -1;
  row_lim = min(row_lim, kend - 1);
  const int nb = (kend + BN - 1) / BN;

  // q row of this lane as f16 (exact for bf16 values within the f16 range)
  f16x8 qf[KS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)t * p.q_st;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qp + s * 16 + lh * 8);
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_h2(__uint_as_float(w[e] << 16), __uint_as_float(w[e] & 0xffff0000u));
      qf[s] = __builtin_bit_cast(f16x8, u32x4{o[0], o[1], o[2], o[3]});
    }
  }

  const unsigned char* kb = p.k + b * p.k_sb + kvh * p.k_sh + (int64_t)k_lo * p.k_st;
  const unsigned char* vb = p.v + b * p.v_sb + kvh * p.v_sh + (int64_t)k_lo * p.v_st;
  // raw dwords of tile j: dword w = i*64 + lane is byte 4w of the tile's
  // rows laid end to end (row r = 4w / RB); rows past kend repeat row kend-1.
  // Byte offsets stay below 2^32: the host limits a range to 2^31 bytes.
  const void* kbs = uniform_ptr(kb);
  const void* vbs = uniform_ptr(vb);
  // rows packed back to back (token stride == row bytes, the usual cache
  // layout): a whole tile is one contiguous byte range, so every load is a
  // scalar base plus the lane's fixed offset 4 * (64 i + lane)
  const bool packed = p.k_st == RB && p.v_st == RB;
  auto load = [&](int j) {
    const uint32_t lk = lds_u32(rawk[j & 1]), lv = lds_u32(rawv[j & 1]);
    if (packed && (j + 1) * BN <= kend) {
      const void* ks = uniform_ptr(kb + (int64_t)j * BN * RB);
      const void* vs = uniform_ptr(vb + (int64_t)j * BN * RB);
#pragma unroll
      for (int i = 0; i < RAW_PL; ++i) {
        dma4(ks, 4u * (uint32_t)(i * 64 + lane), lk + 256u * i);
        dma4(vs, 4u * (uint32_t)(i * 64 + lane), lv + 256u * i);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < RAW_PL; ++i) {
      const int w = i * 64 + lane, r = (4 * w) / RB, c = (4 * w) % RB;
      const int key = min(j * BN + r, kend - 1);
      dma4(kbs, (uint32_t)(key * (uint32_t)p.k_st + c), lk + 256u * i);
      dma4(vbs, (uint32_t)(key * (uint32_t)p.v_st + c), lv + 256u * i);
    }
  };

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  if (nb > 0) load(0);
  for (int j = 0; j < nb; ++j) {
    // tile j has landed; every LDS read of the previous iteration has returned
    // before the next tile's loads may overwrite the other stage
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    if (j + 1 < nb) load(j + 1);  // in flight while this tile is decoded and multiplied
    // decode: chunk c = (key r, 8 values from column 8 * (c % CPR))
    const unsigned char* rkb = reinterpret_cast<const unsigned char*>(rawk[j & 1]);
    const unsigned char* rvb = reinterpret_cast<const unsigned char*>(rawv[j & 1]);
#pragma unroll
    for (int i = 0; i < CH_PL; ++i) {
      const int c = i * 64 + lane, r = c / CPR, kc = c % CPR;
      const int d0 = kc * 8, bb = r * RB + (d0 / 32) * BB;
      *reinterpret_cast<u32x4*>(kt + chunk_at<CPR>(r, kc)) = decode8<FMT>(rkb, bb, d0 % 32);
      *reinterpret_cast<u32x4*>(vt + chunk_at<CPR>(r, kc)) = decode8<FMT>(rvb, bb, d0 % 32);
      // wide heads decode two chunks at a time: hoisting every raw read of the
      // tile ahead of its use would hold 8 registers per chunk (they spill)
      if (D >= 256 && i % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
    // one wave: its own LDS writes are visible to its later LDS reads
    lds_order();
    f32x16 S;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) S = mfma16(row_frag<CPR>(kt, lq, s, lh), qf[s], S);
    // S^T element i: key j*BN + lh*4 + 8*(i/4) + i%4 of this lane's row
    const int key0 = j * BN;
    if (key0 + BN - 1 > row_lim) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key0 + lh * 4 + 8 * (i >> 2) + (i & 3) > row_lim) S[i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[i]);
    // the running max moves only when a score exceeds it by more than 2^8
    // (P <= 256 in f16 meanwhile), so the rescale of O is rare
    const float mnew = fmaxf(m_run, halves_max(mx));
    const bool grow = (mnew - m_run) * p.c > 8.f;  // false when both are -inf
    if (__any(grow)) {
      const float alpha = grow ? ((m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - mnew) * p.c)) : 1.f;
      if (grow) m_run = mnew;
      l_run *= alpha;
      if constexpr (DT >= 8) {
        // wide heads: the accumulator fills the AGPRs; scale each value in
        // place (read, multiply, write back) so that no copy of it is held in
        // VGPRs. The wait covers the last MFMA that wrote an accumulator.
        asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float tmp;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\ts_nop 1\n\tv_mul_f32 %1, %1, %2\n\ts_nop 1\n\t"
                         "v_accvgpr_write_b32 %0, %1"
                         : "+a"(acc[dt][i]), "=&v"(tmp)
                         : "v"(alpha));
          }
      } else {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
      }
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * p.c;
    float P[16], rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      P[i] = __builtin_amdgcn_exp2f(fmaf(S[i], p.c, -mc));
      rs += P[i];
    }
    l_run += rs;
    const f16x8 pb0 = __builtin_bit_cast(
        f16x8, u32x4{pack_h2(P[0], P[1]), pack_h2(P[2], P[3]), pack_h2(P[4], P[5]), pack_h2(P[6], P[7])});
    const f16x8 pb1 = __builtin_bit_cast(
        f16x8, u32x4{pack_h2(P[8], P[9]), pack_h2(P[10], P[11]), pack_h2(P[12], P[13]), pack_h2(P[14], P[15])});
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc[dt] = mfma16(tr_frag<CPR>(vt, 0, dt * 32, lane), pb0, acc[dt]);
      acc[dt] = mfma16(tr_frag<CPR>(vt, 16, dt * 32, lane), pb1, acc[dt]);
    }
  }

  // epilogue: O^T tiles, lane holds row `f`, columns dt*32 + 8*g4 + 4*lh .. +3
  const float lt = halves_sum(l_run);
  const float ms = (m_run == -INFINITY) ? -INFINITY : m_run * p.scale;
  if (!valid) return;
  const int64_t l_off = ((int64_t)b * p.H + h) * p.Tq + t;
  if (p.n_splits > 1) {
    const float pinv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t prow = (int64_t)blockIdx.y * ((int64_t)p.B * p.H * p.Tq) + l_off;
    float* po = p.part_o + prow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + lh * 4;
        *reinterpret_cast<f32x4*>(po + d) = f32x4{acc[dt][g4 * 4] * pinv, acc[dt][g4 * 4 + 1] * pinv,
                                                  acc[dt][g4 * 4 + 2] * pinv, acc[dt][g4 * 4 + 3] * pinv};
      }
    if (lh == 0) p.part_lse[prow] = lt > 0.f ? ms + __builtin_amdgcn_logf(lt) * kLn2 : -INFINITY;
    return;
  }
  float inv, lse;
  if (p.sinks != nullptr) {
    const float sk = p.sinks[h];
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
  uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + b * p.o_sb + h * p.o_sh + (int64_t)t * p.o_st;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = dt * 32 + g4 * 8 + lh * 4;
      *reinterpret_cast<u32x2*>(ob + d) = u32x2{pack_bf2(acc[dt][g4 * 4] * inv, acc[dt][g4 * 4 + 1] * inv),
                                                pack_bf2(acc[dt][g4 * 4 + 2] * inv, acc[dt][g4 * 4 + 3] * inv)};
    }
  if (lh == 0) p.lse[l_off] = lse;
}

template <int FMT, int D>
int launch_cfg(const QkvParams& p, void* stream) {
  hipLaunchKernelGGL((qkv_decode_kernel<FMT, D>), dim3(p.n_rt * p.B * p.Hkv, p.n_splits > 1 ? p.n_splits : 1),
                     dim3(64), 0, reinterpret_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

template <int FMT, int D>
int occ_cfg() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&qkv_decode_kernel<FMT, D>), 64,
                                                   0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

}  // namespace

int launch_qkv(const QkvParams& p, int fmt, int d, void* stream) {
  if (fmt == kFmtQ8 && d == 128) return launch_cfg<kFmtQ8, 128>(p, stream);
  if (fmt == kFmtQ4 && d == 128) return launch_cfg<kFmtQ4, 128>(p, stream);
  if (fmt == kFmtQ8 && d == 256) return launch_cfg<kFmtQ8, 256>(p, stream);
  if (fmt == kFmtQ4 && d == 256) return launch_cfg<kFmtQ4, 256>(p, stream);
  return -1;
}

int occupancy_qkv(int fmt, int d) {
  if (fmt == kFmtQ8 && d == 128) return occ_cfg<kFmtQ8, 128>();
  if (fmt == kFmtQ4 && d == 128) return occ_cfg<kFmtQ4, 128>();
  if (fmt == kFmtQ8 && d == 256) return occ_cfg<kFmtQ8, 256>();
  if (fmt == kFmtQ4 && d == 256) return occ_cfg<kFmtQ4, 256>();
  return 0;
}

}  // namespace attn
