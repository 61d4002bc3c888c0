// Decode attention over a quantized K/V cache for AMD CDNA4 (gfx950).
//
// K and V are stored in llama.cpp's q8_0 or q4_0 block formats (blocks of 32
// values along the head dimension: an fp16 scale, then 32 int8 codes or 16
// bytes of 4-bit codes). The llama.cpp page ("Pins #303") describes the point
// of the in-kernel path: the attention kernel dequantizes the K/V tiles it
// loads, instead of converting the whole cache to f16 on every step.
//
// A wave owns 16 folded query rows (GQA: the g heads x Tq tokens of one kv
// head, e.g. 4 heads x 4 tokens of a multi-sequence decode step), or two such
// row tiles where a kv head has more rows (each decoded K block then feeds
// both tiles' products, so the cache is read and decoded once per 32 rows),
// and walks 32-key tiles with v_mfma_f32_16x16x32_f16:
//
//   raw bytes   each lane loads, straight into registers, the whole blocks it
//               decodes: block (4i + lane/16) of two keys (lane%16 and
//               16 + lane%16), so one lane decodes one key's block end to end
//   S^T = K Q^T the decoded K block is the MFMA's A operand as it stands
//               (the contraction order over d is permuted so that a lane's
//               eight k-elements of step 4i + c are chunk c of its block;
//               q is loaded in the same order); K never goes through LDS
//   softmax     online, base 2, lazy rescale; a query's four lane groups
//               reduce through permlane swaps
//   O^T += V^T P^T  the decoded V block goes to the wave's f16 tile in LDS and
//               comes back as V^T by transposed reads
//
// f16 keeps the decoded values to 11 significant bits (a q8_0 value d*q needs
// up to 18) where bf16 would keep 8; q is converted from bf16 exactly.
//
// A workgroup holds NW waves on the same rows; they take the tiles of its key
// range in turn and merge their (max, sum, O) through LDS at the end, so a
// workgroup writes one result: the output, or with several key ranges (grid
// y) the range's partial result for the split-KV merge.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_params.h"

namespace attn {
namespace {

typedef _Float16 f16_t;
typedef __bf16 bf16_t;
typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef f16_t f16x2 __attribute__((ext_vector_type(2)));
typedef f16_t f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kFmtQ8 = 8, kFmtQ4 = 2;  // the ggml type numbers of q8_0 and q4_0

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// max / sum over a query's four lane groups (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float groups_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float groups_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
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

// The V tile is written as 128-bit chunks and read back by transposed 64-bit
// reads: a compiler barrier keeps these LDS accesses in program order (one
// wave's LDS operations complete in order).
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// 16-byte chunk swizzle of a V tile row of CPR chunks (64 LDS banks): 16
// consecutive rows put one logical chunk in 16 distinct bank groups.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  static_assert(CPR % 16 == 0, "rows of whole 256-byte groups");
  return ((r & 3) << 2) | ((r >> 2) & 3);
}

template <int CPR>
__device__ __forceinline__ int chunk_at(int r, int c) {
  return r * (CPR * 8) + ((c ^ swz<CPR>(r)) << 3);
}

// A operand V^T for output columns c0..c0+15 (lane%16) and keys {4g..4g+3,
// 16+4g..16+4g+3} of the tile (g = lane/16, the keys of the lane's P values):
// each 16-lane group reads a 4-key x 16-column block per transposed read and
// lane i receives column i of it.
template <int CPR>
__device__ __forceinline__ f16x8 v_frag(const f16_t* tile, int c0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int col = c0 + 4 * (i & 3);
  uint32_t w[4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int row = 16 * hh + 4 * g + (i >> 2);
    const f16_t* ptr = tile + row * (CPR * 8) + (((col >> 3) ^ swz<CPR>(row)) << 3) + (col & 7);
    const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)ptr);
    w[2 * hh] = (uint32_t)(uint16_t)t[0] | ((uint32_t)(uint16_t)t[1] << 16);
    w[2 * hh + 1] = (uint32_t)(uint16_t)t[2] | ((uint32_t)(uint16_t)t[3] << 16);
  }
  return __builtin_bit_cast(f16x8, u32x4{w[0], w[1], w[2], w[3]});
}

// Block geometry. A block sits at byte 34 b (q8_0) or 18 b (q4_0) of a row
// whose length is a multiple of 4, so even blocks start 4-byte aligned and odd
// blocks 2 bytes past a dword. A lane loads WIN dwords from the dword at or
// just before its block (2 bytes early for odd blocks, which stays inside the
// row: the previous block's codes) and shifts them by those 2 bytes, which
// gives n[x] = bytes 4x .. 4x+3 of the block: the scale in n[0]'s low half,
// code byte k at byte 2 + k. The window of an even block runs 2 bytes into
// the next block of the same row (the last block of a row is odd).
template <int FMT>
struct Blk {
  static constexpr int BB = FMT == kFmtQ8 ? 34 : 18;  // bytes per block
  static constexpr int WIN = (BB + 2 + 3) / 4;          // dwords loaded per block
};

// Decode one block from its normalised dwords n[] into 16 words of packed f16
// (word m = values 2m, 2m + 1).
//
// Packed f16 arithmetic: a byte b placed under the exponent byte 0x64 is the
// f16 number 1024 + b exactly; one byte permute with 0x64 bytes as its other
// source builds two such numbers, one packed subtract removes the offset
// (1024 + 128 for int8 codes with their sign bit flipped, 1024 + 8 for
// nibbles) and one packed multiply applies the scale (d * code rounded once
// to f16, as the single f32 product rounded to f16 would be).
__device__ __forceinline__ uint32_t code_pair(uint32_t word, int m, f16x2 off, f16x2 d2) {
  // values 2m, 2m+1 sit at bytes 2 + 2m, 3 + 2m: byte 2 and 3 of the word for
  // even m, bytes 0 and 1 for odd m; selector 4 takes byte 0 of the first
  // source (0x64)
  const uint32_t sel = (m & 1) ? 0x04010400u : 0x04030402u;
  const uint32_t bits = __builtin_amdgcn_perm(0x64646464u, word, sel);
  return __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, bits) - off) * d2);
}

template <int FMT>
__device__ __forceinline__ void decode_block(const uint32_t (&n)[Blk<FMT>::WIN], uint32_t (&dec)[16]) {
  constexpr int WIN = Blk<FMT>::WIN;
  const f16x2 d2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(n[0], n[0], 0x01000100u));
  if constexpr (FMT == kFmtQ8) {
    uint32_t c[WIN];
#pragma unroll
    for (int x = 0; x < WIN; ++x) c[x] = n[x] ^ 0x80808080u;  // int8 q -> q + 128 (n[0]'s scale bytes unused)
    const f16x2 off = {(f16_t)1152.f, (f16_t)1152.f};
#pragma unroll
    for (int m = 0; m < 16; ++m) dec[m] = code_pair(c[(m + 1) >> 1], m, off, d2);
  } else {
    // value e < 16: low nibble of code byte e; value e >= 16: high nibble of byte e - 16
    uint32_t lo[WIN], hi[WIN];
#pragma unroll
    for (int x = 0; x < WIN; ++x) {
      lo[x] = n[x] & 0x0f0f0f0fu;
      hi[x] = (n[x] >> 4) & 0x0f0f0f0fu;
    }
    const f16x2 off = {(f16_t)1032.f, (f16_t)1032.f};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      dec[m] = code_pair(lo[(m + 1) >> 1], m, off, d2);
      dec[m + 8] = code_pair(hi[(m + 1) >> 1], m, off, d2);
    }
  }
}

// raw window dwords -> block dwords (shift by sh = 0 or 2 bytes)
template <int WIN>
__device__ __forceinline__ void normalise(const uint32_t (&r)[WIN], uint32_t sh, uint32_t (&n)[WIN]) {
#pragma unroll
  for (int x = 0; x < WIN; ++x) n[x] = __builtin_amdgcn_alignbyte(r[x + 1 < WIN ? x + 1 : x], r[x], sh);
}

// CS = 1: every wave covers all D columns. CS = 2 (512-wide heads, whose
// accumulator, q and raw blocks do not fit one wave): waves come in pairs on
// the same tiles, wave c of a pair takes columns c D/2 .. (c+1) D/2 - 1 for
// both its partial S^T and its output; the pair adds its two partial scores
// through LDS (double-buffered, one workgroup barrier per tile, both waves
// summing in the same order, so they hold identical scores and run identical
// softmax state).
template <int FMT, int D, int NW, int CS, int RT>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW < 4 ? 1 : NW / 4)))
qkv_decode_kernel(const QkvParams p) {
  constexpr int BN = 32;                   // keys per tile
  constexpr int RB = 16 * RT;              // folded rows of the workgroup
  constexpr int BB = Blk<FMT>::BB, WIN = Blk<FMT>::WIN;
  constexpr int DC = D / CS;               // columns of one wave
  constexpr int NBK = DC / 32;             // blocks per row in those columns
  constexpr int BPL = NBK / 4;             // blocks per key a lane decodes
  constexpr int KS = DC / 32;              // S MFMA steps
  constexpr int DT = DC / 16;              // 16-column output tiles
  constexpr int CPR = DC / 8;
  constexpr int NP = NW / CS;              // waves (CS = 1) or pairs (CS = 2) taking tiles in turn
  static_assert(NBK % 4 == 0 && NW <= 16 && NW % CS == 0 && (CS == 1 || CS == 2), "shapes");
  static_assert(CS == 1 || RT == 1, "column pairs hold one row tile");
  // one f16 V tile per wave; after the key loop the same bytes hold the
  // waves' partial outputs (NW x RT x DT x 64 lanes x 16 bytes)
  constexpr int VT_ELEMS = NW * BN * DC, PART_ELEMS = NW * RT * DT * 64 * 8;
  __shared__ __attribute__((aligned(16))) f16_t vt_all[VT_ELEMS > PART_ELEMS ? VT_ELEMS : PART_ELEMS];
  __shared__ float ml_all[NW][RB][2];
  // partial scores of the pairs (CS = 2): [tile parity][wave][lane] x 8 floats
  __shared__ __attribute__((aligned(16))) f32x4 xs_all[CS == 2 ? 2 * NW * 64 * 2 : 1];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ql = lane & 15, lg = lane >> 4;
  const int pr = w / CS, cs = w % CS;      // pair (or wave) and its column half
  f16_t* vt = vt_all + w * (BN * DC);
  const int grp = blockIdx.x / p.n_rt, rt = blockIdx.x % p.n_rt;
  const int b = grp / p.Hkv, kvh = grp % p.Hkv;
  const int rows = p.g * p.Tq;
  const int f0 = rt * RB;
  const int off = p.Tk - p.Tq;
  // row tile r: folded row f0 + 16 r + ql of this lane (head and token
  // recomputed where needed rather than held across the key loop)
  auto row_of = [&](int r, int& h, int& t) -> bool {
    const int f = f0 + 16 * r + ql;
    const int fc = f < rows ? f : rows - 1;
    h = kvh * p.g + fc / p.Tq;
    t = fc % p.Tq;
    return f < rows;
  };

  // keys the workgroup's rows can see, then this workgroup's key range
  int kend = p.Tk;
  if (p.causal) {
    const int f_last = min(f0 + RB, rows) - 1;
    const int t_hi = (f_last / p.Tq != f0 / p.Tq) ? p.Tq - 1 : f_last % p.Tq;
    kend = min(p.Tk, max(0, t_hi + off + 1));
  }
  int k_lo = 0, k_hi = p.Tk;
  if (p.n_splits > 1) {
    k_lo = blockIdx.y * p.split_keys;
    k_hi = min(p.Tk, k_lo + p.split_keys);
  }
  kend = max(0, min(kend, k_hi) - k_lo);
  int row_lim[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int h, t;
    const bool v = row_of(r, h, t);
    row_lim[r] = v ? (p.causal ? min(p.Tk - 1, t + off) : p.Tk - 1) - k_lo : -1;
    row_lim[r] = min(row_lim[r], kend - 1);
  }
  const int nb = (kend + BN - 1) / BN;

  // q rows of this lane as f16, in the permuted contraction order: step s
  // takes values DC cs + 32 (4 (s / 4) + lane/16) + 8 (s % 4) .. + 7
  f16x8 qf[RT][KS];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int h, t;
    row_of(r, h, t);
    const uint16_t* qp =
        reinterpret_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)t * p.q_st + DC * cs;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int d0 = 32 * ((s / 4) * 4 + lg) + 8 * (s % 4);
      const u32x4 wq = *reinterpret_cast<const u32x4*>(qp + d0);
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_h2(__uint_as_float(wq[e] << 16), __uint_as_float(wq[e] & 0xffff0000u));
      qf[r][s] = __builtin_bit_cast(f16x8, u32x4{o[0], o[1], o[2], o[3]});
    }
  }

  const unsigned char* kb = p.k + b * p.k_sb + kvh * p.k_sh + (int64_t)k_lo * p.k_st;
  const unsigned char* vb = p.v + b * p.v_sb + kvh * p.v_sh + (int64_t)k_lo * p.v_st;
  const uint32_t kst = (uint32_t)p.k_st, vst = (uint32_t)p.v_st;
  const uint32_t sh = (lg & 1) * 2;
  // window start of the lane's block i within a row
  uint32_t boff[BPL];
#pragma unroll
  for (int i = 0; i < BPL; ++i) boff[i] = (uint32_t)((NBK * cs + i * 4 + lg) * BB) - sh;

  // raw windows of tile j: [key half][block][dword]; keys past kend repeat
  // key kend - 1 (their scores are masked). Byte offsets stay below 2^31: the
  // host limits one head's rows to that.
  uint32_t rk[2][BPL][WIN], rv[2][BPL][WIN];
  auto load = [&](const unsigned char* base, uint32_t st, int j, uint32_t (&r)[2][BPL][WIN]) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const uint32_t key = (uint32_t)min(j * BN + kh * 16 + ql, kend - 1);
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        const uint32_t* wp = reinterpret_cast<const uint32_t*>(base + (key * st + boff[i]));
#pragma unroll
        for (int x = 0; x < WIN; ++x) r[kh][i][x] = wp[x];
      }
    }
  };

  f32x4 acc[RT][DT];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[r][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }

  // With CS = 2 every wave runs the same number of iterations (the pair
  // barrier is the workgroup's): iterations past nb do no work.
  const int iters = CS == 1 ? (nb > pr ? (nb - pr + NP - 1) / NP : 0) : (nb + NP - 1) / NP;
  if (pr < nb) {
    load(kb, kst, pr, rk);
    load(vb, vst, pr, rv);
  }
  for (int it = 0; it < iters; ++it) {
    const int j = pr + it * NP;
    const bool live = j < nb;  // always true with CS = 1
    const bool more = j + NP < nb;
    // S^T for the tile's two 16-key halves and every row tile, K decoded
    // once straight into the A operand
    f32x4 S[RT][2];
#pragma unroll
    for (int r = 0; r < RT; ++r) S[r][0] = S[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (live) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          uint32_t n[WIN], dec[16];
          normalise<WIN>(rk[kh][i], sh, n);
          decode_block<FMT>(n, dec);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const f16x8 ka = __builtin_bit_cast(f16x8, u32x4{dec[4 * c], dec[4 * c + 1], dec[4 * c + 2], dec[4 * c + 3]});
#pragma unroll
            for (int r = 0; r < RT; ++r) S[r][kh] = mfma16(ka, qf[r][4 * i + c], S[r][kh]);
          }
        }
      }
      if (more) load(kb, kst, j + NP, rk);  // in flight while V is decoded and multiplied
    }
    if constexpr (CS == 2) {
      // the pair's scores: own half + partner half, always half 0 first
      f32x4* xs = xs_all + (it & 1) * (NW * 64 * 2);
      xs[(w * 64 + lane) * 2] = S[0][0];
      xs[(w * 64 + lane) * 2 + 1] = S[0][1];
      __syncthreads();
      const f32x4 o0 = xs[((w ^ 1) * 64 + lane) * 2], o1 = xs[((w ^ 1) * 64 + lane) * 2 + 1];
      if (cs == 0) {
        S[0][0] += o0;
        S[0][1] += o1;
      } else {
        S[0][0] = o0 + S[0][0];
        S[0][1] = o1 + S[0][1];
      }
    }
    if (!live) continue;
    // V: decoded into the wave's f16 tile (row = key, the lane's blocks)
    lds_order();
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        uint32_t n[WIN], dec[16];
        normalise<WIN>(rv[kh][i], sh, n);
        decode_block<FMT>(n, dec);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *reinterpret_cast<u32x4*>(vt + chunk_at<CPR>(kh * 16 + ql, 4 * (i * 4 + lg) + c)) =
              u32x4{dec[4 * c], dec[4 * c + 1], dec[4 * c + 2], dec[4 * c + 3]};
      }
    if (more) load(vb, vst, j + NP, rv);
    // scores of this lane: query ql of each row tile, keys j*BN + 16 kh + 4 lg + e
    const int key0 = j * BN;
    f16x8 pb[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (key0 + BN - 1 > row_lim[r]) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (key0 + 16 * kh + 4 * lg + e > row_lim[r]) S[r][kh][e] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(S[r][0][0], S[r][0][1]), fmaxf(S[r][0][2], S[r][0][3])),
                       fmaxf(fmaxf(S[r][1][0], S[r][1][1]), fmaxf(S[r][1][2], S[r][1][3])));
      // the running max moves only when a score exceeds it by more than 2^8
      // (P <= 256 in f16 meanwhile), so the rescale of O is rare
      const float mnew = fmaxf(m_run[r], groups_max(mx));
      const bool grow = (mnew - m_run[r]) * p.c > 8.f;  // false when both are -inf
      if (__any(grow)) {
        const float alpha =
            grow ? ((m_run[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run[r] - mnew) * p.c)) : 1.f;
        if (grow) m_run[r] = mnew;
        l_run[r] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[r][dt] *= alpha;
      }
      const float mc = (m_run[r] == -INFINITY) ? 0.f : m_run[r] * p.c;
      float P[8];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 4; ++e) P[4 * kh + e] = __builtin_amdgcn_exp2f(fmaf(S[r][kh][e], p.c, -mc));
      l_run[r] += ((P[0] + P[1]) + (P[2] + P[3])) + ((P[4] + P[5]) + (P[6] + P[7]));
      pb[r] = __builtin_bit_cast(
          f16x8, u32x4{pack_h2(P[0], P[1]), pack_h2(P[2], P[3]), pack_h2(P[4], P[5]), pack_h2(P[6], P[7])});
    }
    lds_order();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f16x8 va = v_frag<CPR>(vt, dt * 16, lane);
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[r][dt] = mfma16(va, pb[r], acc[r][dt]);
    }
  }

  // merge the waves (pairs) over the key range: lane holds query ql of each
  // row tile, columns DC cs + dt*16 + 4 lg .. +3; wave (pr, cs) finishes the
  // output tiles dt = pr, pr + NP, ... of its column half for every row
  // tile. The two waves of a pair hold the same row state.
  float M[RT], L[RT];
  constexpr int DW = (DT + NP - 1) / NP;
  float fac[RT][NP];
  f32x4* part = reinterpret_cast<f32x4*>(vt_all);  // [NW][RT][DT][64]
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    M[r] = m_run[r];
    L[r] = groups_sum(l_run[r]);
  }
  if constexpr (NP > 1) {
    __syncthreads();  // every wave is done with its V tile
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) part[((w * RT + r) * DT + dt) * 64 + lane] = acc[r][dt];
      if (lg == 0) {
        ml_all[w][16 * r + ql][0] = m_run[r];
        ml_all[w][16 * r + ql][1] = L[r];
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float Mr = -INFINITY;
#pragma unroll
      for (int u = 0; u < NP; ++u) Mr = fmaxf(Mr, ml_all[u * CS + cs][16 * r + ql][0]);
      float Lr = 0.f;
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const float mu = ml_all[u * CS + cs][16 * r + ql][0];
        fac[r][u] = (mu == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mu - Mr) * p.c);
        Lr += fac[r][u] * ml_all[u * CS + cs][16 * r + ql][1];
      }
      M[r] = Mr;
      L[r] = Lr;
    }
  }
  // the x-th output tile of this wave for row tile r, unnormalised
  auto tile_sum = [&](int r, int x) -> f32x4 {
    if constexpr (NP == 1) {
      return acc[r][x];
    } else {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NP; ++u) s += fac[r][u] * part[(((u * CS + cs) * RT + r) * DT + pr + x * NP) * 64 + lane];
      return s;
    }
  };

#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int h, t;
    if (!row_of(r, h, t)) continue;
    const float ms = (M[r] == -INFINITY) ? -INFINITY : M[r] * p.scale;
    const int64_t l_off = ((int64_t)b * p.H + h) * p.Tq + t;
    if (p.n_splits > 1) {
      const float pinv = L[r] > 0.f ? 1.f / L[r] : 0.f;
      const int64_t prow = (int64_t)blockIdx.y * ((int64_t)p.B * p.H * p.Tq) + l_off;
      float* po = p.part_o + prow * D + DC * cs;
#pragma unroll
      for (int x = 0; x < DW; ++x) {
        if (NP > 1 && pr + x * NP >= DT) break;
        *reinterpret_cast<f32x4*>(po + (pr + x * NP) * 16 + 4 * lg) = tile_sum(r, x) * pinv;
      }
      if (lg == 0 && w == 0) p.part_lse[prow] = L[r] > 0.f ? ms + __builtin_amdgcn_logf(L[r]) * kLn2 : -INFINITY;
      continue;
    }
    float inv, lse;
    if (p.sinks != nullptr) {
      const float sk = p.sinks[h];
      const float Mx = fmaxf(ms, sk);
      if (Mx == -INFINITY) {
        inv = 0.f;
        lse = -INFINITY;
      } else {
        const float fa = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((ms - Mx) * kLog2e);
        const float es = (sk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((sk - Mx) * kLog2e);
        const float den = L[r] * fa + es;
        inv = den > 0.f ? fa / den : 0.f;
        lse = den > 0.f ? Mx + __builtin_amdgcn_logf(den) * kLn2 : -INFINITY;
      }
    } else {
      inv = L[r] > 0.f ? 1.f / L[r] : 0.f;
      lse = L[r] > 0.f ? ms + __builtin_amdgcn_logf(L[r]) * kLn2 : -INFINITY;
    }
    uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + b * p.o_sb + h * p.o_sh + (int64_t)t * p.o_st + DC * cs;
#pragma unroll
    for (int x = 0; x < DW; ++x) {
      if (NP > 1 && pr + x * NP >= DT) break;
      const f32x4 o = tile_sum(r, x);
      *reinterpret_cast<u32x2*>(ob + (pr + x * NP) * 16 + 4 * lg) =
          u32x2{pack_bf2(o[0] * inv, o[1] * inv), pack_bf2(o[2] * inv, o[3] * inv)};
    }
    if (lg == 0 && w == 0) p.lse[l_off] = lse;
  }
}

// waves per workgroup: every wave a CU can hold (three per SIMD at d 128, two
// at d 256), so one workgroup per CU covers the longest key range; with more
// row tiles a wave holds more accumulators and fewer waves fit
template <int FMT, int D, int RT>
constexpr int waves_of() {
  if constexpr (D == 128) return RT == 1 ? 12 : 8;
  else if constexpr (D == 256) return RT == 1 ? 8 : 4;
  else return 6;
}

// column halves per wave pair: 512-wide heads split their columns over two waves
template <int D>
constexpr int cs_of() {
  return D == 512 ? 2 : 1;
}

template <int FMT, int D, int RT>
int launch_cfg(const QkvParams& p, void* stream) {
  constexpr int NW = waves_of<FMT, D, RT>();
  hipLaunchKernelGGL((qkv_decode_kernel<FMT, D, NW, cs_of<D>(), RT>),
                     dim3(p.n_rt * p.B * p.Hkv, p.n_splits > 1 ? p.n_splits : 1), dim3(64 * NW), 0,
                     reinterpret_cast<hipStream_t>(stream), p);
  return (int)hipGetLastError();
}

template <int FMT, int D, int RT>
int occ_cfg() {
  int n = 0;
  constexpr int NW = waves_of<FMT, D, RT>();
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&qkv_decode_kernel<FMT, D, NW, cs_of<D>(), RT>), 64 * NW, 0) !=
      hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

template <int FMT, int D>
int launch_rt(const QkvParams& p, int rt, void* stream) {
  if constexpr (D == 512) {
    return rt == 1 ? launch_cfg<FMT, D, 1>(p, stream) : -1;
  } else {
    if (rt == 1) return launch_cfg<FMT, D, 1>(p, stream);
    if constexpr (D == 128 || FMT == kFmtQ4)
      if (rt == 2) return launch_cfg<FMT, D, 2>(p, stream);
    return -1;
  }
}

template <int FMT, int D>
int occ_rt(int rt) {
  if constexpr (D == 512) {
    return rt == 1 ? occ_cfg<FMT, D, 1>() : 0;
  } else {
    if (rt == 1) return occ_cfg<FMT, D, 1>();
    if constexpr (D == 128 || FMT == kFmtQ4)
      if (rt == 2) return occ_cfg<FMT, D, 2>();
    return 0;
  }
}

}  // namespace

int qkv_row_tiles(int fmt, int d, int rows) {
  // two row tiles (8 waves, two per SIMD) where a kv head has more than 16
  // folded rows; four (4 waves, one per SIMD) measured slower on long caches.
  // q8_0's wider raw blocks leave no room for two at d 256, the column pairs
  // of d 512 none at all
  if (d == 512 || rows <= 16) return 1;
  if (d == 256 && fmt != kFmtQ4) return 1;
  return 2;
}

int launch_qkv(const QkvParams& p, int fmt, int d, int rt, void* stream) {
  if (fmt == kFmtQ8 && d == 128) return launch_rt<kFmtQ8, 128>(p, rt, stream);
  if (fmt == kFmtQ4 && d == 128) return launch_rt<kFmtQ4, 128>(p, rt, stream);
  if (fmt == kFmtQ8 && d == 256) return launch_rt<kFmtQ8, 256>(p, rt, stream);
  if (fmt == kFmtQ4 && d == 256) return launch_rt<kFmtQ4, 256>(p, rt, stream);
  if (fmt == kFmtQ8 && d == 512) return launch_rt<kFmtQ8, 512>(p, rt, stream);
  if (fmt == kFmtQ4 && d == 512) return launch_rt<kFmtQ4, 512>(p, rt, stream);
  return -1;
}

int occupancy_qkv(int fmt, int d, int rt) {
  if (fmt == kFmtQ8 && d == 128) return occ_rt<kFmtQ8, 128>(rt);
  if (fmt == kFmtQ4 && d == 128) return occ_rt<kFmtQ4, 128>(rt);
  if (fmt == kFmtQ8 && d == 256) return occ_rt<kFmtQ8, 256>(rt);
  if (fmt == kFmtQ4 && d == 256) return occ_rt<kFmtQ4, 256>(rt);
  if (fmt == kFmtQ8 && d == 512) return occ_rt<kFmtQ8, 512>(rt);
  if (fmt == kFmtQ4 && d == 512) return occ_rt<kFmtQ4, 512>(rt);
  return 0;
}

}  // namespace attn
