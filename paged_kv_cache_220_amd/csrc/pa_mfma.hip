// Matrix-core PagedAttention decode partition kernel (gfx950, wave64).
//
// Same work unit as the vector kernel: one wavefront per (sequence, KV head,
// context partition), all G <= 16 query heads of the KV head together, so
// every K/V tile is read once per KV head. The online-softmax state of the
// PagedAttention kernel pseudocode (vLLM page: running max m, running sum l,
// rescaled o, output o / l) stays in registers. Here the two contractions of
// a grouped decode step run on v_mfma_f32_16x16x32_{bf16,f16}:
//   S^T[token][head] = K^T[token][d] . Q^T[d][head]   (contract over head_dim)
//   O^T[d][head]    += V[d][token]  . P^T[token][head] (contract over tokens)
// with heads on the 16 MFMA columns (columns >= G carry zero queries).
//
// The cache tile is [head_dim][16 tokens] with tokens fastest, which suits PV
// directly (a 128-bit load is 8 tokens of one row) but not QK, whose operand
// wants several head_dim values of one token per lane. Each lane takes 8
// rows x 4 tokens and transposes them in registers with v_perm_b32, feeding
// 4 MFMAs (one per token of the quartet). The MFMA k index may map to
// head_dim in any order as long as the Q operand uses the same order, so lane
// group c takes rows 32*kstep + 4*i + c. For bf16 those are 64-bit loads
// straight from HBM, and every load instruction covers whole 128-byte lines.
// For fp8 the 4-token pieces are only 4 bytes, so the K tile is first copied
// into LDS as whole rows by buffer-to-LDS copies, and the pieces are read
// from there.
//
// A tile is 64 tokens = 4 physical blocks. MFMA row (quartet) q = 4c + r of
// the QK step holds block (c >> 1) + 2 * (r >> 1), tokens 8 * (c & 1) +
// 4 * (r & 1) + j, j = 0..3 (one MFMA per j). With that placement the QK
// accumulator already sits where the PV step needs P: lane (c, head) holds
// the 8 consecutive tokens 8 * (c & 1) .. +7 of block (c >> 1) + 2 * hh for
// PV instruction hh, which are exactly the tokens of its 128-bit V load.
// So P moves from the score accumulator to the PV operand inside the lane;
// the only cross-lane traffic is the max over the four lane groups per tile
// and the final sum of l.
//
// Token slots at or past the partition end are selected out: their scores
// become -inf, and their V values are zeroed before the MFMA (0 * NaN would
// poison the sum). Logical blocks past the partition end are not looked up in
// the table; the tile's first block stands in and is masked.
//
// fp8 KV (E5M2 here, E4M3 below): an E5M2 byte is the top byte of the binary16 of the same
// value, so v_perm_b32 widens K and V to fp16 exactly and the f16 MFMA runs
// with q in binary16. Each query column is first scaled by a power of two that
// puts its largest |q| in [2^14, 2^15) (the scores are scaled back in fp32), so
// every bf16 q converts exactly down to 2^-28 of the column's maximum, and no
// finite q overflows. Per-block V scales are split into mantissa and exponent:
// the mantissa multiplies P, the exponent joins the score (see softmax), so P
// stays in [0, 2) whatever the scales.
// bf16 KV: bf16 MFMA with q exact. In both, P enters the PV product as two
// 16-bit operands (the rounded weight and its rounding residual), so the
// weights carry about twice the operand precision into the fp32 accumulator.

#include <hip/hip_ext.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"



namespace pa {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kD = 128;       // head_dim handled by this kernel
// s_waitcnt operand (gfx9 encoding: vmcnt[3:0] at bits 3:0 and vmcnt[5:4] at
// bits 15:14, expcnt at 6:4, lgkmcnt at 11:8) that waits for vmcnt == 0 and
// leaves the other counters unconstrained.
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);
// The same operand waiting for vmcnt <= n (n < 64).
constexpr int vmcnt_wait(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// Word 3 of a raw buffer resource on gfx9-family chips (32-bit data format,
// no swizzle, no index stride): offsets are plain bytes from the base.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kTile = 64;     // tokens per tile
constexpr int kKSteps = kD / 32;

template <int KDT> struct Mfma;

template <> struct Mfma<kBF16> {
  using op_t = bf16x8;
  using kload_t = u32x2;   // 4 tokens of one row
  using vload_t = u32x4;   // 8 tokens of one row
  static constexpr int kBits = 16;   // storage bits per value
  static __device__ __forceinline__ f32x4 mma(op_t a, op_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // Operand holding K[rows 2p, 2p+1 of the 8 loaded rows][token j of the quartet].
  static __device__ __forceinline__ op_t k_operand(const kload_t (&r)[8], int j) {
    const int w = j >> 1;
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    u32x4 x;
    x[0] = __builtin_amdgcn_perm(r[1][w], r[0][w], sel);
    x[1] = __builtin_amdgcn_perm(r[3][w], r[2][w], sel);
    x[2] = __builtin_amdgcn_perm(r[5][w], r[4][w], sel);
    x[3] = __builtin_amdgcn_perm(r[7][w], r[6][w], sel);
    return __builtin_bit_cast(op_t, x);
  }
  static __device__ __forceinline__ op_t v_operand(vload_t x) { return __builtin_bit_cast(op_t, x); }
  // Zero the token slots at index >= nvalid (0..8) of an 8-token V segment.
  static __device__ __forceinline__ vload_t mask_v(vload_t x, int nvalid) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = (2 * w < nvalid) ? 0x0000FFFFu : 0u;
      const uint32_t hi = (2 * w + 1 < nvalid) ? 0xFFFF0000u : 0u;
      x[w] &= (lo | hi);
    }
    return x;
  }
  // q is bf16 already: the operand is its bits, packed two per register
  // (bf16 has float32's exponent range, so q needs no rescaling).
  static constexpr bool kRescaleQ = false;
  static __device__ __forceinline__ op_t q_operand(const uint32_t (&qb)[8], int) {
    u32x4 x;
#pragma unroll
    for (int w = 0; w < 4; ++w) x[w] = qb[2 * w] | (qb[2 * w + 1] << 16);
    return __builtin_bit_cast(op_t, x);
  }
  // P as a sum of two operands: hi = round(p), lo = round(p - hi), so the PV
  // product keeps about 16 significant bits of each weight.
  // Pairs are rounded together (one packed conversion each for hi and lo);
  // the rounded pair widens back to float by bit placement.
  static __device__ __forceinline__ void p_operands(const float (&p)[8], op_t& hi, op_t& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 x = {p[2 * i], p[2 * i + 1]};
      const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
      const f32x2 hx = {__builtin_bit_cast(float, hw << 16), __builtin_bit_cast(float, hw & 0xFFFF0000u)};
      h[i] = hw;
      l[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x - hx, bf16x2));
    }
    hi = __builtin_bit_cast(op_t, h);
    lo = __builtin_bit_cast(op_t, l);
  }
};

template <> struct Mfma<kE5M2> {
  using op_t = f16x8;
  using kload_t = uint32_t;  // 4 tokens of one row
  using vload_t = u32x2;     // 8 tokens of one row
  static constexpr int kBits = 8;
  static __device__ __forceinline__ f32x4 mma(op_t a, op_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // binary16 bits = e5m2 byte << 8; selector 0x0C yields a zero byte.
  static __device__ __forceinline__ op_t k_operand(const kload_t (&r)[8], int j) {
    const uint32_t sel = 0x0Cu | (uint32_t(j) << 8) | (0x0Cu << 16) | (uint32_t(4 + j) << 24);
    u32x4 x;
    x[0] = __builtin_amdgcn_perm(r[1], r[0], sel);
    x[1] = __builtin_amdgcn_perm(r[3], r[2], sel);
    x[2] = __builtin_amdgcn_perm(r[5], r[4], sel);
    x[3] = __builtin_amdgcn_perm(r[7], r[6], sel);
    return __builtin_bit_cast(op_t, x);
  }
  static __device__ __forceinline__ op_t v_operand(vload_t x) {
    u32x4 y;
    y[0] = __builtin_amdgcn_perm(x[0], x[0], 0x010C000Cu);
    y[1] = __builtin_amdgcn_perm(x[0], x[0], 0x030C020Cu);
    y[2] = __builtin_amdgcn_perm(x[1], x[1], 0x010C000Cu);
    y[3] = __builtin_amdgcn_perm(x[1], x[1], 0x030C020Cu);
    return __builtin_bit_cast(op_t, y);
  }
  static __device__ __forceinline__ vload_t mask_v(vload_t x, int nvalid) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t m = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) m |= (4 * w + b < nvalid) ? (0xFFu << (8 * b)) : 0u;
      x[w] &= m;
    }
    return x;
  }
  // q (bf16) times 2^shift, rounded to binary16. The caller picks the shift
  // per query column so that its largest |q| lands in [2^14, 2^15): every
  // element within 2^-28 of that maximum is then a normal binary16, exact
  // (bf16 carries 8 significant bits, binary16 11), and nothing overflows.
  // The scores are scaled back by 2^-shift in float32.
  static constexpr bool kRescaleQ = true;
  static __device__ __forceinline__ op_t q_operand(const uint32_t (&qb)[8], int shift) {
    op_t o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = static_cast<_Float16>(__builtin_amdgcn_ldexpf(bf16_bits_to_f32(qb[i]), shift));
    return o;
  }
  static __device__ __forceinline__ void p_operands(const float (&p)[8], op_t& hi, op_t& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 x = {p[2 * i], p[2 * i + 1]};
      const half2_t hh = __builtin_convertvector(x, half2_t);
      h[i] = __builtin_bit_cast(uint32_t, hh);
      l[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x - __builtin_convertvector(hh, f32x2), half2_t));
    }
    hi = __builtin_bit_cast(op_t, h);
    lo = __builtin_bit_cast(op_t, l);
  }
};

// int4 KV: two's-complement codes, two tokens per byte (the even token in the
// low nibble), so a K piece of 4 tokens is 2 bytes and a V piece of 8 tokens
// 4 bytes. The operands carry u = code ^ 8 = code + 8 (0..15) as a binary16
// subnormal: the bit pattern u is the value u * 2^-24 exactly, and the pattern
// 16u (the nibble one place up) is 16u * 2^-24, still subnormal. So widening
// is one mask per pair of values (and a shift for half of K's); the offset
// and the power of two are taken out of the fp32 results instead:
//   score = 2^24 / s_j * (u-product) - 8 * sum_d q[d]   (s_j = 1 or 16: kKShift)
//   o     = 2^24 * (u-product)       - 8 * sum_t p[t]
// with the sums over the f16 q values and over the P values fed to the MFMA.
// The per-block scales are applied to the scores (K) and to P (V).
template <> struct Mfma<kI4> {
  using op_t = f16x8;
  using kload_t = uint16_t;  // 4 tokens of one row
  using vload_t = uint32_t;  // 8 tokens of one row
  static constexpr int kBits = 4;
  static constexpr float kOffset = 8.f;          // u = code + 8
  static constexpr float kUnit = 16777216.f;     // 2^24: one subnormal binary16 step
  // QK instruction for token j of a quartet produces s_j times the product
  static constexpr float kKScale[4] = {1.f, 16.f, 1.f, 16.f};
  static __device__ __forceinline__ f32x4 mma(op_t a, op_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // token j of rows 2p (low half) and 2p + 1 (high half): nibble j of each half
  // at bits 0..3 (j = 0, 2) or 4..7 (j = 1, 3)
  static __device__ __forceinline__ op_t k_operand(const kload_t (&r)[8], int j) {
    u32x4 x;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t w = (uint32_t(r[2 * p]) | (uint32_t(r[2 * p + 1]) << 16)) ^ 0x88888888u;
      x[p] = (j < 2 ? w : w >> 8) & ((j & 1) ? 0x00F000F0u : 0x000F000Fu);
    }
    return __builtin_bit_cast(op_t, x);
  }
  // V: the 8 tokens of a row segment enter the MFMA in the order kVTok, half
  // of them (kVHigh) at scale 16 (nibble left at bits 4..7); P is fed in the
  // same order with those weights divided by 16, so each product is
  // p * u * 2^-24. Two masks and a shift per 8 values, no byte permutes.
  static constexpr int kVTok[8] = {0, 4, 1, 5, 2, 6, 3, 7};
  static constexpr bool kVHigh[8] = {false, false, true, true, false, false, true, true};
  static __device__ __forceinline__ op_t v_operand(vload_t x) {
    const uint32_t w = x ^ 0x88888888u;
    const uint32_t s = w >> 8;
    u32x4 y;
    y[0] = w & 0x000F000Fu;   // tokens 0, 4
    y[1] = w & 0x00F000F0u;   // tokens 1, 5 (x16)
    y[2] = s & 0x000F000Fu;   // tokens 2, 6
    y[3] = s & 0x00F000F0u;   // tokens 3, 7 (x16)
    return __builtin_bit_cast(op_t, y);
  }
  static __device__ __forceinline__ vload_t mask_v(vload_t x, int nvalid) {
    return nvalid >= 8 ? x : (nvalid <= 0 ? 0u : x & ((1u << (4 * nvalid)) - 1u));   // code 0 = value 0
  }
  static constexpr bool kRescaleQ = true;
  static __device__ __forceinline__ op_t q_operand(const uint32_t (&qb)[8], int shift) {
    return Mfma<kE5M2>::q_operand(qb, shift);
  }
  static __device__ __forceinline__ void p_operands(const float (&p)[8], op_t& hi, op_t& lo) {
    Mfma<kE5M2>::p_operands(p, hi, lo);
  }
};

// Query columns. Query position qi (0 <= qi < q_len) of query head kvh*G + h
// is "virtual head" v = qi*G + h, placed on MFMA column v % 16 of column group
// v / 16; NCG groups cover G * q_len <= 16 * NCG. All groups share each K and
// V operand, so a tile is read once whatever the number of queries. With one
// query (decode) and G <= 16 there is a single group.
// One work item: partition `part` of sequence s for KV head kvh, all its columns.
// fp8-e4m3 KV: gfx950 converts two OCP E4M3 codes to two binary16 values in
// one instruction; every E4M3 value (subnormals included, |x| <= 448) is a
// normal binary16, so the widening is exact. Otherwise as for E5M2.
template <> struct Mfma<kE4M3> {
  using op_t = f16x8;
  using kload_t = uint32_t;  // 4 tokens of one row
  using vload_t = u32x2;     // 8 tokens of one row
  static constexpr int kBits = 8;
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  template <bool kHiWord>   // codes in bytes 2, 3 (else 0, 1) -> two binary16 values
  static __device__ __forceinline__ uint32_t cvt2(uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, kHiWord));
  }
  static __device__ __forceinline__ f32x4 mma(op_t a, op_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ op_t k_operand(const kload_t (&r)[8], int j) {
    const uint32_t sel = uint32_t(j) | (uint32_t(4 + j) << 8) | 0x0C0C0000u;   // token j of rows 2p, 2p+1
    u32x4 x;
    x[0] = cvt2<false>(__builtin_amdgcn_perm(r[1], r[0], sel));
    x[1] = cvt2<false>(__builtin_amdgcn_perm(r[3], r[2], sel));
    x[2] = cvt2<false>(__builtin_amdgcn_perm(r[5], r[4], sel));
    x[3] = cvt2<false>(__builtin_amdgcn_perm(r[7], r[6], sel));
    return __builtin_bit_cast(op_t, x);
  }
  static __device__ __forceinline__ op_t v_operand(vload_t x) {
    u32x4 y;
    y[0] = cvt2<false>(x[0]);
    y[1] = cvt2<true>(x[0]);
    y[2] = cvt2<false>(x[1]);
    y[3] = cvt2<true>(x[1]);
    return __builtin_bit_cast(op_t, y);
  }
  static __device__ __forceinline__ vload_t mask_v(vload_t x, int nvalid) { return Mfma<kE5M2>::mask_v(x, nvalid); }
  static constexpr bool kRescaleQ = true;
  static __device__ __forceinline__ op_t q_operand(const uint32_t (&qb)[8], int shift) {
    return Mfma<kE5M2>::q_operand(qb, shift);
  }
  static __device__ __forceinline__ void p_operands(const float (&p)[8], op_t& hi, op_t& lo) {
    Mfma<kE5M2>::p_operands(p, hi, lo);
  }
};

// STREAM: K/V loads bypass the caches (each tile is read once per call). Work
// items that are one of several query blocks of a KV head (four column
// groups) load through the caches instead, so the sibling blocks that read
// the same tiles at about the same time on the same XCD can hit in them.
// BSCALE: the cache carries per-(block, KV head) scales (int4 always, fp8
// optionally); the kernel without them keeps the registers their products take.
// STAGES > 0: tile sharing. The NW waves of the workgroup take NW consecutive
// query blocks of the item (query block qb * NW + wave) and walk the same
// tiles; each K/V tile is copied once into a ring of STAGES LDS stages by all
// waves together and every wave reads its operands from there. STAGES == 0:
// the NW waves split the tiles of one query block and merge their states.
template <int KDT, int NCG, int NW, bool STREAM, bool BSCALE, int STAGES>
__device__ __forceinline__ void partition_item(const Args& a, int group, int s, int kvh, int part, int qb) {
  using M = Mfma<KDT>;
  using op_t = typename M::op_t;
  using kload_t = typename M::kload_t;
  using vload_t = typename M::vload_t;
  constexpr int BS = kBlockSize;
  constexpr int64_t kRowBytes = BS * M::kBits / 8;         // one head_dim row of a block tile

  const int L = clamp_len(a, s);
  const int QL = a.q_len;
  const int GV = group * QL;                               // virtual heads of this KV head
  constexpr bool kShare = STAGES > 0;
  const int P = a.partition_tokens;
  const int nparts = L > 0 ? (L + P - 1) / P : 1;
  if (part >= nparts) return;
  const int tok0 = part * P;
  const int tok1 = min(L, tok0 + P);
  // Tokens below this bound are inside the partition and inside every query's
  // causal window (query 0 of the last QL positions attends t < L - QL + 1);
  // columns past the last (position, head) pair carry zero queries and are
  // never written, so they need no selection either.
  const int full_lim = min(tok1, L - QL + 1);

  // NW waves share the item: without tile sharing wave w takes tiles w, w + NW, ...
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __builtin_assume(wave >= 0 && wave < NW);   // lets the copy assignment below fold
  // first virtual head of this wave's query block
  const int v0 = kShare ? 16 * NCG * (qb * NW + wave) : 16 * kMaxColumnGroups * qb;
  const int lane = threadIdx.x & 63;
  const int c = lane >> 4;   // lane group: k slots of the operands, rows 4c..4c+3 of results
  const int n = lane & 15;   // MFMA row of A (quartet / head_dim row) and column of B (virtual head)

  // Q^T operands: lane (c, n) of group cg holds q[query qi][head h][32*ks + 4*i + c],
  // i = 0..7. Columns past the last virtual head read a valid row and zero it, so
  // all loads issue back to back without a branch between them. The loads and
  // the conversion to operands are apart: the plain loop issues its first K/V
  // tile in between, so that q's latency and the tile's overlap.
  constexpr bool kLdsK = !kShare && (M::kBits < 16 || NCG == 2);
  constexpr bool kPlain = !kShare && !kLdsK;
  // P enters PV as hi + lo (about 16 significant bits per weight) in bf16
  // decode (one column group). With several query positions, where the
  // matrix cores and the vector ALU bound the kernel, and in fp8 and int4
  // decode, where the shorter tile step lets the next loads go out sooner
  // (int4: its tile step is compute-bound), it enters as hi alone (bf16: 8
  // bits, binary16: 11), which halves the PV products. The error of an
  // output is then at most 2^-9 (2^-12) of sum_i p_i |v_i|, the attention
  // over |V|.
  constexpr bool kTwoPartP = NCG == 1 && M::kBits == 16;
  // bf16 tile sharing reads its K operands from LDS with gfx950's
  // transposing read (ds_read_b64_tr_b16), which hands each lane one token's
  // values of four rows, so no register transpose follows. The read fixes
  // which tokens can share an instruction's rows: rows 4q..4q+3 are four
  // consecutive tokens. The tokens of the QK results are then those of the
  // other kernels with the roles of result register r and instruction j
  // exchanged (score (r, j) of lane group c is token 16 ((c >> 1) + 2 (j >> 1))
  // + 8 (c & 1) + 4 (j & 1) + r), which leaves the V operands as they are and
  // only reorders P.
  constexpr bool kTrK = kShare && KDT == kBF16 && !BSCALE;
  op_t qop[NCG][kKSteps];
  int lim[NCG];                // tokens the column's query may attend: t < lim
  float qsum[NCG];             // int4: sum_d q[d] of the column
  float qss[NCG];              // score scale of the column: scale * k_scale * log2(e) * 2^-(q shift)
  uint32_t qraw[NCG][kKSteps][8];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int v = v0 + 16 * cg + n;
    const bool col_ok = v < GV;
    const int qi = col_ok ? v / group : 0;
    const int h = col_ok ? v - qi * group : 0;
    lim[cg] = col_ok ? L - QL + 1 + qi : 0;
    const uint16_t* qh = static_cast<const uint16_t*>(a.q) +
                         (((int64_t)s * QL + qi) * a.num_heads + (int64_t)kvh * group + h) * kD;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
      for (int i = 0; i < 8; ++i) qraw[cg][ks][i] = qh[32 * ks + 4 * i + c];
    }
  }
  auto make_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const bool col_ok = v0 + 16 * cg + n < GV;
      // binary16 operands: the column's largest |q| (bf16 magnitudes order as
      // integers; the column spans the four lane groups) sets a power of two
      // that brings it into [2^14, 2^15); the score scale undoes it in float32.
      int shift = 0;
      uint32_t qmax = 0;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          qraw[cg][ks][i] = col_ok ? qraw[cg][ks][i] : 0u;
          qmax = max(qmax, qraw[cg][ks][i] & 0x7FFFu);
        }
      }
      if constexpr (M::kRescaleQ) {
        qmax = max(qmax, (uint32_t)__shfl_xor((int)qmax, 16, 64));
        qmax = max(qmax, (uint32_t)__shfl_xor((int)qmax, 32, 64));
        shift = 15 - __builtin_amdgcn_frexp_expf(bf16_bits_to_f32(qmax));   // max in [2^(e-1), 2^e)
      }
      // (held at the smallest normal float: a row of nothing but bf16 subnormals
      // would otherwise scale its scores by 0)
      qss[cg] = M::kRescaleQ ? fmaxf(__builtin_amdgcn_ldexpf(a.score_scale, -shift), 1.17549435e-38f) : a.score_scale;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qop[cg][ks] = M::q_operand(qraw[cg][ks], shift);
      if constexpr (KDT == kI4) {
        // sum over head_dim of the binary16 q values the MFMA uses
        float qs = 0.f;
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
          for (int i = 0; i < 8; ++i) qs += static_cast<float>(qop[cg][ks][i]);
        }
        qs += shfl_xor_f32(qs, 16);
        qs += shfl_xor_f32(qs, 32);
        qsum[cg] = qs;
      }
    }
  };
  if constexpr (!kPlain) make_q();

  // This lane's block (0..3 within a tile) and token offset for the K loads.
  const int kblk = (n >> 3) + 2 * ((n >> 1) & 1);
  const int ktok = 8 * ((n >> 2) & 1) + 4 * (n & 1);
  // Byte offsets inside a block tile of this KV head.
  const int64_t head_off = (int64_t)kvh * kD * kRowBytes;
  const int64_t blk_bytes = a.block_stride * M::kBits / 8;
  const char* kbase = static_cast<const char*>(a.k) + head_off;
  const char* vbase = static_cast<const char*>(a.v) + head_off;
  const int32_t* table = a.tables + (int64_t)s * a.max_blocks;
  const int nblk_part = (tok1 + BS - 1) / BS;   // logical blocks that hold partition tokens

  float m_run[NCG];          // running max per column (log2 domain), same in all lane groups
  float l_run[NCG];          // this lane group's share of the running sum
  float pv_run[NCG];         // int4: its share of the running sum of the P values fed to PV
  f32x4 oacc[NCG][8];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    m_run[cg] = -INFINITY;
    l_run[cg] = 0.f;
    pv_run[cg] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[cg][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int first = tok0 + (kShare ? 0 : wave) * kTile;
  // Tiles of the partition, and how many of them lie wholly inside the
  // partition and inside every query's window (they need no selection; the
  // others are the partition's last tiles). The full tiles are visited in an
  // order rotated by a per-sequence offset: sequences that share prefix blocks
  // (the same physical blocks at the same logical positions) then reach them
  // at different times, so the tiles the caches serve and the tiles that come
  // from HBM are mixed throughout the launch instead of every item reading the
  // shared prefix first. All KV heads of a sequence keep one order (a block's
  // KV heads lie side by side in memory), and the offset depends only on the
  // sequence and partition, so every kernel variant and schedule visits the
  // same order.
  const int ntiles_all = (tok1 - tok0 + kTile - 1) / kTile;
  const int nfull_all = max(0, min(ntiles_all, (full_lim - tok0) / kTile));
  const uint32_t item_hash = ((uint32_t)(s * a.max_parts + part)) * 2654435761u;
  // (four bf16 column groups split over two waves keep the plain order: the
  // rotation's registers would spill there, and no other variant is held to
  // their bits)
  constexpr bool kRotate = !(kPlain && NCG == 4 && NW > 1);
  const int rot = kRotate && nfull_all > 0 ? (int)((item_hash >> 16) % (uint32_t)nfull_all) : 0;
  auto tstart = [&](const int k) __attribute__((always_inline)) {   // start token of tile k in visiting order
    int j = k;
    if (k < nfull_all) {
      j = k + rot;
      if (j >= nfull_all) j -= nfull_all;
    }
    return tok0 + j * kTile;
  };

  // K slots in LDS (one per wave) for the kernels that stage K tiles there:
  // fp8 (whole-row copies instead of 4-byte pieces) and two column groups
  // (one wave per SIMD: the next tile's K copy then overlaps this tile's
  // compute at no register cost). Four bf16 groups have no registers left
  // for the staged loop and load K directly.
  constexpr int kTileBlk = kD * kRowBytes;   // one block tile of one KV head
  constexpr int kSlotBlk = kTileBlk + 64;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kLdsK ? NW : 1][kLdsK ? 4 * kSlotBlk : 16];
  // Tile sharing: stage x holds the K tile (4 block slots) then the V tile.
  // One array per stage: distinct objects, which the compiler knows apart
  // (below).
  constexpr int kStageBytes = kShare ? 8 * kSlotBlk : 16;
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds1[STAGES > 1 ? kStageBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds2[STAGES > 2 ? kStageBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds3[STAGES > 3 ? kStageBytes : 16];
  auto stage = [&](auto S) __attribute__((always_inline)) -> uint8_t* {
    constexpr int x = decltype(S)::value;
    if constexpr (x == 0) return kv_lds0;
    else if constexpr (x == 1) return kv_lds1;
    else if constexpr (x == 2) return kv_lds2;
    else return kv_lds3;
  };
  // One tile's K and V registers.
  struct Tile {
    kload_t kr[kKSteps][8];
    vload_t vr[8][2];
  };
  // Vector-memory instructions of one tile's V load (one per vr element).
  constexpr int kVLoadInsts = 8 * 2;
  static_assert(sizeof(Tile::vr) == kVLoadInsts * sizeof(vload_t), "one load per V register group");
  auto ld = [&](auto* ptr) __attribute__((always_inline)) {
    if constexpr (STREAM) return __builtin_nontemporal_load(ptr);
    else return *ptr;
  };
  // K loads: 4 k-steps x 8 rows, 4 tokens each; V loads: 8 row tiles x 2
  // token halves, 8 tokens each. K/V bytes are used once per call, so they are
  // loaded non-temporally (streamed past the caches).
  auto load_k = [&](Tile& T, int32_t ik) __attribute__((always_inline)) {
    const int64_t kb_off = clamp_block(a, ik) * blk_bytes;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = 32 * ks + 4 * i + c;
        T.kr[ks][i] = ld(reinterpret_cast<const kload_t*>(kbase + kb_off + d * kRowBytes + ktok * M::kBits / 8));
      }
    }
  };
  auto load_v = [&](Tile& T, int32_t iv0, int32_t iv1) __attribute__((always_inline)) {
    const int64_t vb_offs[2] = {clamp_block(a, iv0) * blk_bytes, clamp_block(a, iv1) * blk_bytes};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int d = 16 * dt + n;
        T.vr[dt][hh] = ld(reinterpret_cast<const vload_t*>(vbase + vb_offs[hh] + d * kRowBytes + 8 * (c & 1) * M::kBits / 8));
      }
    }
  };
  auto load_tile = [&](Tile& T, int32_t ik, int32_t iv0, int32_t iv1) __attribute__((always_inline)) {
    load_k(T, ik);
    load_v(T, iv0, iv1);
  };
  // ---- S^T = K^T Q^T: MFMA j covers token j of every quartet; the K operand
  // is shared by all column groups
  auto qk = [&](Tile& T, f32x4 (&sacc)[NCG][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const op_t kop = M::k_operand(T.kr[ks], j);
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
          sacc[cg][j] = M::mma(kop, qop[cg][ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[cg][j]);
      }
    }
  };
  // ---- online softmax of column group cg over this tile; P leaves as two
  // 16-bit PV operands per instruction hh (rounded weight and its residual)
  // ksc[x] / vsc[x]: per-block K / V scale of the tile's block (c >> 1) + 2x
  // (1 without per-block scales); quartets r = 2x, 2x + 1 and PV instruction x
  // of this lane lie in that block.
  //
  // With per-block V scales, the weight fed to PV for a token of block x is
  // p * vsc[x], which a 16-bit operand cannot hold for every scale (it
  // overflows above about 2^15 and loses bits below 2^-14). So vsc[x] is split
  // into vm[x] * 2^ve[x] with vm in [1, 2): the power of two joins the score
  // (s' = s + ve, exact in the log2 domain) and the running max follows s',
  // so the largest fed weight of the state is 2^0 * vm, whatever the scales.
  // PV receives 2^(s' - m) * vm = 2^(s - m) * vsc, and the running sum adds
  // 2^(s' - m) * 2^-ve = 2^(s - m): the state (m, l, o) keeps its meaning with
  // m the reference of both sums, and o / l is unchanged.
  auto softmax = [&](auto edge, const int cg, const f32x4 (&sg)[4], const int t0, op_t (&phi)[2],
                     op_t (&plo)[2], const float (&ksc)[2], const float (&vsc)[2])
      __attribute__((always_inline)) {
    const int nval = min(tok1, lim[cg]) - t0;   // this column's tokens in the tile (may be <= 0)
    // Plain scores (no int4 offset, no per-block scales) are product * ka with
    // ka > 0; the others are one fma each, kept in sc ([r][j], -inf outside
    // the window).
    constexpr bool kPlainScores = KDT != kI4 && !BSCALE;
    float sc[4][4];
    float tmax = -INFINITY;
    float ka[2], kb[2];                         // score = product * ka + kb, per block of the lane
    float vm[2];                                // V scale's mantissa (1 without per-block scales)
    int ve[2];                                  // and its exponent
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      if constexpr (BSCALE) {
        ve[x] = __builtin_amdgcn_frexp_expf(vsc[x]) - 1;
        vm[x] = 2.f * __builtin_amdgcn_frexp_mantf(vsc[x]);
      } else {
        ve[x] = 0;
        vm[x] = 1.f;
      }
      if constexpr (KDT == kI4) {
        ka[x] = qss[cg] * ksc[x] * Mfma<kI4>::kUnit;
        kb[x] = -(qss[cg] * ksc[x]) * (Mfma<kI4>::kOffset * qsum[cg]) + (float)ve[x];
      } else {
        ka[x] = qss[cg] * ksc[x];
        kb[x] = (float)ve[x];
      }
    }
    // Only a tile that reaches past the partition end or a query's window
    // has tokens to select out (the caller's wave-uniform test, taken once
    // per tile as a compile-time branch so full tiles carry no selects).
    const bool select = decltype(edge)::value && t0 + kTile > full_lim;
    auto valid = [&](int r, int j) __attribute__((always_inline)) {
      if constexpr (kTrK) return 16 * ((c >> 1) + 2 * (j >> 1)) + 8 * (c & 1) + 4 * (j & 1) + r < nval;
      return 16 * ((c >> 1) + 2 * (r >> 1)) + 8 * (c & 1) + 4 * (r & 1) + j < nval;
    };
    if constexpr (kPlainScores) {
      // one positive factor for the whole column: the largest score is that
      // factor times the largest product, bit for bit (rounding is monotonic)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) tmax = fmaxf(tmax, (select && !valid(r, j)) ? -INFINITY : sg[j][r]);
      }
      tmax *= ka[0];
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (KDT == kI4) sc[r][j] = fmaf(sg[j][r], ka[r >> 1] * (1.f / Mfma<kI4>::kKScale[j]), kb[r >> 1]);
          else sc[r][j] = fmaf(sg[j][r], ka[r >> 1], kb[r >> 1]);
          if (select) sc[r][j] = valid(r, j) ? sc[r][j] : -INFINITY;
          tmax = fmaxf(tmax, sc[r][j]);
        }
      }
    }
    tmax = fmaxf(tmax, shfl_xor_f32(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f32(tmax, 32));
    const float m_new = fmaxf(m_run[cg], tmax);
    // A column with no token yet keeps m = -inf. Subtracting 0 instead of -inf
    // then makes every weight and the rescale 2^-inf = 0, so its state stays
    // zero and -inf - -inf is never formed.
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run[cg] - m_use);
    m_run[cg] = m_new;
    float psum[2] = {0.f, 0.f};                 // per block of the lane
    float p[4][4];
    // The sums take the tokens in one order in every kernel: with the
    // exchanged roles of r and j (kTrK) the loops run over (j, r).
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = kTrK ? b : a, j = kTrK ? a : b;
        // Plain scores: the exponent is one fma of the product (the max above
        // used the rounded product), written out so every tile and every
        // kernel variant takes the same arithmetic. Scaled scores already
        // are one fma each.
        float arg;
        if constexpr (kPlainScores) {
          arg = fmaf(sg[j][r], ka[r >> 1], -m_use);
          if (select) arg = valid(r, j) ? arg : -INFINITY;
        } else {
          arg = sc[r][j] - m_use;
        }
        p[r][j] = __builtin_amdgcn_exp2f(arg);
        psum[a >> 1] += p[r][j];
      }
    }
    if constexpr (BSCALE)
      l_run[cg] = l_run[cg] * alpha + (__builtin_amdgcn_ldexpf(psum[0], -ve[0]) + __builtin_amdgcn_ldexpf(psum[1], -ve[1]));
    else
      l_run[cg] = l_run[cg] * alpha + (psum[0] + psum[1]);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[cg][dt] *= alpha;
    // PV instruction hh takes quartets r = 2hh, 2hh+1 (token i of the lane's
    // 8-token segment is p[2hh + i / 4][i % 4])
    float pv_lo = 0.f, pv_hi = 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float pv[8];
      if constexpr (KDT == kI4) {
        // int4: tokens in the V operand's order, the scale-16 ones divided by 16
        // (exactly); the sums add exactly the rounded values PV receives (the
        // empty asm keeps the compiler from fusing the product into the sum,
        // which it would do in some instantiations and not in others)
        const float vs16 = vm[hh] * 0.0625f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = Mfma<kI4>::kVTok[k];
          pv[k] = p[2 * hh + (i >> 2)][i & 3] * (Mfma<kI4>::kVHigh[k] ? vs16 : vm[hh]);
          // with hi alone, PV receives binary16(pv): sum that (the operand
          // conversion of an exact binary16 value then changes nothing)
          if constexpr (!kTwoPartP) pv[k] = static_cast<float>(static_cast<_Float16>(pv[k]));
          asm("" : "+v"(pv[k]));
          if (Mfma<kI4>::kVHigh[k]) pv_hi += pv[k];
          else pv_lo += pv[k];
        }
      } else if constexpr (kTrK) {
        // slots 0-3 are rows r = 0..3 of instruction 2hh, 4-7 those of 2hh + 1
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = p[i & 3][2 * hh + (i >> 2)] * vm[hh];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = p[2 * hh + (i >> 2)][i & 3] * vm[hh];
      }
      M::p_operands(pv, phi[hh], plo[hh]);
    }
    if constexpr (KDT == kI4) pv_run[cg] = fmaf(pv_run[cg], alpha, fmaf(pv_hi, 16.f, pv_lo));
  };
  // V values of token slots at or past the partition end are zeroed: their
  // weights are 0, but 0 * NaN would poison the sum.
  auto mask_tail = [&](auto edge, Tile& T, const int t0) __attribute__((always_inline)) {
    const int nvalid = tok1 - t0;   // tokens of this tile inside the partition (may exceed 64)
    if (decltype(edge)::value && nvalid < kTile) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int seg = 16 * ((c >> 1) + 2 * hh) + 8 * (c & 1);
        const int nv = min(8, max(0, nvalid - seg));
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) T.vr[dt][hh] = M::mask_v(T.vr[dt][hh], nv);
      }
    }
  };
  // One tile: QK, then `after_qk` (the K registers are free from here on),
  // then softmax and O^T += V P^T. With V operands used as loaded (bf16) each
  // column group's PV follows its softmax, so only one group's P is live;
  // widened fp8 V operands are instead shared by all groups' MFMAs.
  auto tile_step = [&](auto edge, Tile& T, const int t0, auto&& after_qk, const float (&ksc)[2],
                       const float (&vsc)[2]) __attribute__((always_inline)) {
    f32x4 sacc[NCG][4];
    qk(T, sacc);
    after_qk();
    mask_tail(edge, T, t0);
    if constexpr (M::kBits == 16) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        op_t phi[2], plo[2];
        softmax(edge, cg, sacc[cg], t0, phi, plo, ksc, vsc);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const op_t vop = M::v_operand(T.vr[dt][hh]);
            oacc[cg][dt] = M::mma(vop, phi[hh], oacc[cg][dt]);
            if constexpr (kTwoPartP) oacc[cg][dt] = M::mma(vop, plo[hh], oacc[cg][dt]);
          }
        }
      }
    } else {
      op_t phi[NCG][2], plo[NCG][2];
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) softmax(edge, cg, sacc[cg], t0, phi[cg], plo[cg], ksc, vsc);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const op_t vop = M::v_operand(T.vr[dt][hh]);
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) {
            oacc[cg][dt] = M::mma(vop, phi[cg][hh], oacc[cg][dt]);
            if constexpr (kTwoPartP) oacc[cg][dt] = M::mma(vop, plo[cg][hh], oacc[cg][dt]);
          }
        }
      }
    }
  };

  // Stage reads address the stage as its array plus this lane's offset plus a
  // constant. The empty asm keeps the lane's offset one value, so that the
  // compiler does not spread its terms over a chain of address steps: the
  // stage reads are then traced to their stage array (the trace has a depth
  // limit), and the compiler holds a read only for the copies into that
  // stage.
  auto lane_offset = [](int x) __attribute__((always_inline)) {
    asm("" : "+v"(x));
    return x;
  };

  // One tile of the tile-sharing kernels with at most two column groups per
  // wave (two waves per SIMD): operands are read from the LDS stage `st` as
  // they are used (K a k-step at a time, V one 8-token row segment at a time)
  // and the other wave on the SIMD covers the LDS latency. Per column the
  // arithmetic and its order are those of tile_step.
  auto share_tile = [&](auto edge, const uint8_t* st, const int t0, const float (&ksc)[2],
                        const float (&vsc)[2]) __attribute__((always_inline)) {
    f32x4 sacc[NCG][4];
    if constexpr (kTrK) {
      // Operand of instruction j, k-step ks for lane (n, c): rows 32 ks + 4 i
      // + c (i = 0..7, the order q's operand uses) of the token of row n. In
      // the transposing read a lane gets slot (its lane % 4) of the 4-element
      // pieces that lanes (its lane / 4) + 4 k (k = 0..3) of its 16-lane group
      // load. So lane n loads row 32 ks + 4 (n / 4) + c (+ 16 for i = 4..7) at
      // the 4 tokens of row group q = n % 4 (block (q >> 1) + 2 (j >> 1),
      // from token 8 (q & 1) + 4 (j & 1)), and receives rows 32 ks + 4 k + c
      // of its own row's token.
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;
      const int q = n & 3;
      const int klane = lane_offset((q >> 1) * kSlotBlk + (4 * (n >> 2) + c) * kRowBytes + 8 * (q & 1) * 2);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kc = 2 * (j >> 1) * kSlotBlk + 32 * ks * kRowBytes + 4 * (j & 1) * 2;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(st + (klane + kc)));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(st + (klane + (kc + 16 * kRowBytes))));
          const op_t kop = __builtin_bit_cast(op_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg)
            sacc[cg][j] = M::mma(kop, qop[cg][ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[cg][j]);
        }
      }
    } else {
      const int klane = lane_offset(kblk * kSlotBlk + c * kRowBytes + ktok * M::kBits / 8);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        kload_t kr[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
          kr[r] = *reinterpret_cast<const kload_t*>(st + (klane + (32 * ks + 4 * r) * kRowBytes));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const op_t kop = M::k_operand(kr, j);
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg)
            sacc[cg][j] = M::mma(kop, qop[cg][ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[cg][j]);
        }
      }
    }
    op_t phi[NCG][2], plo[NCG][2];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) softmax(edge, cg, sacc[cg], t0, phi[cg], plo[cg], ksc, vsc);
    const int nvalid = tok1 - t0;   // tokens of this tile inside the partition (may exceed 64)
    const int vlane = lane_offset((c >> 1) * kSlotBlk + n * kRowBytes + 8 * (c & 1) * M::kBits / 8);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int nv = min(8, max(0, nvalid - (16 * ((c >> 1) + 2 * hh) + 8 * (c & 1))));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int vc = (4 + 2 * hh) * kSlotBlk + 16 * dt * kRowBytes;
        vload_t x = *reinterpret_cast<const vload_t*>(st + (vlane + vc));
        if (decltype(edge)::value && nvalid < kTile) x = M::mask_v(x, nv);   // 0 * NaN would poison the sum
        const op_t vop = M::v_operand(x);
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
          oacc[cg][dt] = M::mma(vop, phi[cg][hh], oacc[cg][dt]);
          if constexpr (kTwoPartP) oacc[cg][dt] = M::mma(vop, plo[cg][hh], oacc[cg][dt]);
        }
      }
    }
  };

  // Helpers of the LDS-staged loops. The four block ids of a tile are the
  // same for the whole wave. They (and the per-block scales) are read through
  // the constant address space, so they become scalar loads even where the
  // compiler cannot tell that the loop's LDS copies leave that memory alone.
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  typedef const __attribute__((address_space(4))) int32_t* cint_ptr_t;
  typedef const __attribute__((address_space(4))) float* cflt_ptr_t;
  const cint_ptr_t ctable = (cint_ptr_t)table;
  const int last_blk = nblk_part - 1;
  auto ids_at = [&](int t, int32_t (&ib)[4]) __attribute__((always_inline)) {
    const int b0 = min(t / BS, last_blk);
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) ib[blk] = clamp_block(a, ctable[b0 + blk < nblk_part ? b0 + blk : b0]);
  };
  // Per-block scales of a tile (the same for the whole wave).
  constexpr bool bscaled = BSCALE;
  auto uniform_f = [](float x) __attribute__((always_inline)) {   // keep wave-uniform values in scalar registers
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
  };
  auto scales_at = [&](const int32_t (&ib)[4], float (&kb)[4], float (&vb)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int64_t at = (int64_t)__builtin_amdgcn_readfirstlane(ib[blk]) * a.num_kv_heads + kvh;
      kb[blk] = bscaled ? uniform_f(((cflt_ptr_t)a.k_bscale)[at]) : 1.f;
      vb[blk] = bscaled ? uniform_f(((cflt_ptr_t)a.v_bscale)[at]) : 1.f;
    }
  };
  // This lane's two scales of a tile: block (c >> 1) + 2x for x = 0, 1.
  auto lane_scales = [&](const float (&b)[4], float (&x)[2]) __attribute__((always_inline)) {
    x[0] = (c >> 1) == 0 ? b[0] : b[1];
    x[1] = (c >> 1) == 0 ? b[2] : b[3];
  };

  if constexpr (kShare) {
    // Tile sharing. A tile's K and V (4 block tiles each) land in one LDS
    // stage through buffer-to-LDS copies of 1 KiB (16 bytes per lane), dealt
    // round robin to the NW waves, STAGES - 1 tiles ahead of use. Before tile
    // i each wave waits for its own copies of it; the workgroup barrier that
    // follows covers the other waves' copies, and also tells that every wave
    // is done with the stage of tile i - 1, which then takes tile
    // i + STAGES - 1. Each wave reads its K pieces and V rows from the stage
    // and runs the tile for its own query block.
    //
    // Tile i uses stage i % STAGES, and the loop holds one copy of the tile
    // step per stage, so every copy and every LDS read names its stage at
    // compile time. The compiler then tells the stage being read from the one
    // being filled and lets the next tile's copies run under this tile's
    // compute; with a stage index known only at run time it holds each tile's
    // first LDS read until every copy in flight has landed.
    constexpr int kCpb = kTileBlk / 1024;     // copies per block tile
    constexpr int kCopies = 8 * kCpb;         // K and V of 4 blocks
    constexpr int kPer = kCopies / NW;        // copies per wave per tile
    static_assert(kCopies % NW == 0, "tile copies must split evenly over the waves");
    static_assert(STAGES >= 2 && STAGES <= 4, "two to four stages");
    const int ntiles = (tok1 - tok0 + kTile - 1) / kTile;
    const bool active = v0 < GV;              // wave-uniform: this wave's query block exists
    auto issue = [&](auto S, int i) __attribute__((always_inline)) {   // tile i into stage S
      int32_t ib[4];
      ids_at(tstart(i), ib);
      uint8_t* st = stage(S);
#pragma unroll
      for (int y = 0; y < kPer; ++y) {
        const int x = y * NW + wave;          // copy x: cache kv, block blk, KiB pc of the block tile
        const int kv = x / (4 * kCpb), blk = (x / kCpb) % 4, pc = x % kCpb;
        int32_t id = ib[0];   // wave-uniform selects (mostly folded), no branches
#pragma unroll
        for (int b = 1; b < 4; ++b) id = blk == b ? ib[b] : id;
        id = __builtin_amdgcn_readfirstlane(id);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>((kv ? vbase : kbase) + id * blk_bytes), 0, kTileBlk, kRawBufferWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(st + (4 * kv + blk) * kSlotBlk + pc * 1024), 16,
                                                 lane * 16 + pc * 1024, 0, 0, STREAM ? 2 : 0);   // 2: non-temporal
      }
    };
    // Prologue: tiles 0 .. STAGES - 2. A partition with fewer tiles copies its
    // last tile again (into a stage no tile uses), so that the number of
    // copies after the q loads is fixed; the loop's waits then count the
    // extra copies as later ones and stay on the safe side.
    if (ntiles > 0) {   // the same for every wave of the item (an empty sequence has none)
      static_for<STAGES - 1>([&](auto S) __attribute__((always_inline)) { issue(S, min(S(), ntiles - 1)); });
      // tile i, which sits in stage S = i % STAGES
      auto step = [&](auto edge, auto S, const int i) __attribute__((always_inline)) {
        constexpr int kS = decltype(S)::value;
        const int t0 = tstart(i);
        // own copies of tile i: everything but those of the later tiles in flight
        const int ahead = min(STAGES - 2, ntiles - 1 - i);
        if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * kPer));
        else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_wait(kPer));
        else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (i + STAGES - 1 < ntiles) issue(std::integral_constant<int, (kS + STAGES - 1) % STAGES>{}, i + STAGES - 1);
        __builtin_amdgcn_sched_barrier(0);
        if (active) {
          float kb[4], vb[4], ksc[2], vsc[2];
          if constexpr (BSCALE) {
            int32_t ib[4];
            ids_at(t0, ib);
            scales_at(ib, kb, vb);
            lane_scales(kb, ksc);
            lane_scales(vb, vsc);
          } else {
            ksc[0] = ksc[1] = vsc[0] = vsc[1] = 1.f;
          }
          const uint8_t* st = stage(S);
          if constexpr (NCG <= 2) {
            share_tile(edge, st, t0, ksc, vsc);
            return;
          }
          const int klane = lane_offset(kblk * kSlotBlk + c * kRowBytes + ktok * M::kBits / 8);
          const int vlane = lane_offset((c >> 1) * kSlotBlk + n * kRowBytes + 8 * (c & 1) * M::kBits / 8);
          Tile T;
#pragma unroll
          for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
              T.kr[ks][r] = *reinterpret_cast<const kload_t*>(st + (klane + (32 * ks + 4 * r) * kRowBytes));
          }
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
              T.vr[dt][hh] = *reinterpret_cast<const vload_t*>(st + (vlane + ((4 + 2 * hh) * kSlotBlk + 16 * dt * kRowBytes)));
          }
          tile_step(edge, T, t0, []() __attribute__((always_inline)) {}, ksc, vsc);
        }
      };
      // Tiles wholly inside the partition and every query's window first (no
      // selects), then the rest: two loops, so full tiles carry no selection
      // and each loop keeps its own register allocation. A loop that may
      // start in the middle of a round of stages first runs the steps up to
      // the round's end; each pass of the loop then runs one step per stage
      // in stage order. (The steps of different stages stay apart in the
      // code: were they merged, the merged reads would address either stage
      // and wait for every copy in flight.)
      int i = 0;
      auto run = [&](auto edge, auto aligned, const int end) __attribute__((always_inline)) {
        if constexpr (!decltype(aligned)::value) {
          static_for<STAGES - 1>([&](auto S) __attribute__((always_inline)) {
            constexpr int kS = decltype(S)::value + 1;
            if (i < end && i % STAGES == kS) {
              step(edge, std::integral_constant<int, kS>{}, i);
              ++i;
            }
          });
        }
        while (i < end) {
          static_for<STAGES>([&](auto S) __attribute__((always_inline)) {
            if (i < end) {
              step(edge, S, i);
              ++i;
            }
          });
        }
      };
      run(std::false_type{}, std::true_type{}, nfull_all);
      run(std::true_type{}, std::false_type{}, ntiles);
    }
    // every wave is past its last stage read: the stages take the outputs of
    // single-partition bf16 items below
    if constexpr (M::kBits == 16) {
      if (nparts == 1) __builtin_amdgcn_s_barrier();
    }
  } else if constexpr (kLdsK) {
    // Staged K. A K tile is 4 block tiles of 128 rows x 16 tokens; it lands in
    // this wave's LDS slot through buffer-to-LDS copies of whole rows
    // (16 bytes per lane, each instruction reading 1 KiB contiguous), and QK
    // reads each lane's 4-token pieces back from LDS. (For fp8, loading those
    // 4-byte pieces straight from HBM touches half of every 128-byte line per
    // instruction and runs the memory pipeline 25 % slower.) Block slots are
    // 64 bytes apart beyond the tile so the four blocks of a read fall in
    // different LDS banks.
    //
    // Pipeline: K of the next tile is issued right after this tile's QK (its
    // slot is free again) and V of the next tile right after PV (into the V
    // registers PV has released). The wait before reading a K tile from LDS
    // leaves that tile's V loads (issued after its K copies) in flight, so V
    // arrives under QK and the softmax. The four block ids of a tile are the
    // same for the whole wave; they are fetched two tiles ahead.
    //
    // The copies are buffer loads with one resource per block tile (base =
    // the tile, size = its bytes), not global ones: the compiler counts those
    // in issue order with the V loads and waits for V before PV with the K
    // copies of the next tile still in flight, while a global-to-LDS load in
    // flight makes it wait for every outstanding load. The explicit wait
    // before the K reads does not depend on the compiler tracing those reads
    // to the slot array (its own waits after such copies do).
    uint8_t* kslot = &k_lds[wave][0];
    const uint8_t* krow = kslot + kblk * kSlotBlk + c * kRowBytes + ktok * M::kBits / 8;   // + row bytes * (32 ks + 4 i)
    // With copy false the resources hold no bytes: the loads touch no memory
    // (out of range) and only keep the loads per tile the same on every path,
    // which lets the compiler count exactly in its waits for V.
    auto load_k_lds = [&](const int32_t (&ib)[4], const bool copy) __attribute__((always_inline)) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        // (ids and sizes are wave-uniform; readfirstlane keeps the resource in
        // scalar registers)
        const int32_t id = __builtin_amdgcn_readfirstlane(ib[blk]);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(kbase + id * blk_bytes), 0, __builtin_amdgcn_readfirstlane(copy ? kTileBlk : 0),
            kRawBufferWord3);
#pragma unroll
        for (int part = 0; part < kTileBlk / 1024; ++part)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(kslot + blk * kSlotBlk + part * 1024), 16,
                                                   lane * 16 + part * 1024, 0, 0,
                                                   STREAM ? 2 : 0);   // 2: non-temporal
      }
    };
    auto load_v_ids = [&](Tile& T, const int32_t (&ib)[4]) __attribute__((always_inline)) {
      load_v(T, (c >> 1) == 0 ? ib[0] : ib[1], (c >> 1) == 0 ? ib[2] : ib[3]);
    };
    if (first < tok1) {
      Tile T;
      int32_t icur[4], inext[4];
      float kb_cur[4], vb_cur[4], kb_next[4], vb_next[4];
      ids_at(tstart(wave), icur);
      ids_at(tstart(wave + NW), inext);
      scales_at(icur, kb_cur, vb_cur);
      load_k_lds(icur, true);
      load_v_ids(T, icur);
      __builtin_amdgcn_sched_barrier(0);
      auto step = [&](auto edge, const int k) __attribute__((always_inline)) {
        const int t0 = tstart(k);
        const bool more = k + NW < ntiles_all;
        scales_at(inext, kb_next, vb_next);   // the next tile's, a tile ahead of use
        float ksc[2], vsc[2];
        lane_scales(kb_cur, ksc);
        lane_scales(vb_cur, vsc);
        // The K copies into LDS are vector-memory operations, and the only
        // ones issued after them are this tile's V loads: waiting until at
        // most those are outstanding completes the copies.
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(kVLoadInsts));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            T.kr[ks][i] = *reinterpret_cast<const kload_t*>(krow + (32 * ks + 4 * i) * kRowBytes);
        }
        auto next_k = [&]() __attribute__((always_inline)) {
          __builtin_amdgcn_sched_barrier(0);
          if (more) ids_at(tstart(k + 2 * NW), icur);
          load_k_lds(inext, more);
          __builtin_amdgcn_sched_barrier(0);
        };
        tile_step(edge, T, t0, next_k, ksc, vsc);
        __builtin_amdgcn_sched_barrier(0);
        // After the last tile the loads read block 0 (in range, unused), so
        // that every path through the loop issues the same loads.
        int32_t vids[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) vids[blk] = more ? inext[blk] : 0;
        load_v_ids(T, vids);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          inext[blk] = icur[blk];
          kb_cur[blk] = kb_next[blk];
          vb_cur[blk] = vb_next[blk];
        }
      };
      int k = wave;   // full tiles first, then the ones that need selection
      for (; k < nfull_all; k += NW) step(std::false_type{}, k);
      for (; k < ntiles_all; k += NW) step(std::true_type{}, k);
      // The last tile's empty copies target this wave's slot, which the
      // epilogue may reuse: let them finish.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
  } else {
    // Plain loop: K and V straight into registers, one tile in flight per
    // wave. This lane's K-load block is kblk of the tile and its V-load blocks
    // (c >> 1) and (c >> 1) + 2; the ids of the next tile are fetched (scalar)
    // behind this tile's loads.
    auto pick = [&](const int32_t (&ib)[4], int j) __attribute__((always_inline)) {
      const int32_t x = (j & 1) ? ib[1] : ib[0];
      const int32_t y = (j & 1) ? ib[3] : ib[2];
      return (j & 2) ? y : x;
    };
    int32_t ib[4] = {0, 0, 0, 0};
    Tile T;
    auto issue = [&](int k) __attribute__((always_inline)) {   // tile k (its ids in ib), then the ids of k + NW
      load_tile(T, pick(ib, kblk), pick(ib, c >> 1), pick(ib, (c >> 1) + 2));
      if (k + NW < ntiles_all) ids_at(tstart(k + NW), ib);
    };
    if (first < tok1) {   // a wave without tiles needs no q operands
      ids_at(tstart(wave), ib);
      issue(wave);
      make_q();
      __builtin_amdgcn_sched_barrier(0);
      auto step = [&](auto edge, const int k) __attribute__((always_inline)) {
        constexpr float kOnes[2] = {1.f, 1.f};
        tile_step(edge, T, tstart(k), []() __attribute__((always_inline)) {}, kOnes, kOnes);
        __builtin_amdgcn_sched_barrier(0);
        if (k + NW < ntiles_all) issue(k + NW);
        __builtin_amdgcn_sched_barrier(0);
      };
      int k = wave;   // full tiles first, then the ones that need selection
      for (; k < nfull_all; k += NW) step(std::false_type{}, k);
      for (; k < ntiles_all; k += NW) step(std::true_type{}, k);
    }
  }

  // ---- epilogue: lane (c, n) of group cg holds O^T[16*dt + 4*c + r][virtual head 16*cg + n]
  if constexpr (KDT == kI4) {
    // o = 2^24 * (offset-code product) - 8 * (sum of the P values fed to PV)
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      float pv_tot = pv_run[cg];
      pv_tot += shfl_xor_f32(pv_tot, 16);
      pv_tot += shfl_xor_f32(pv_tot, 32);
      const float off = Mfma<kI4>::kOffset * pv_tot;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[cg][dt][e] = fmaf(oacc[cg][dt][e], Mfma<kI4>::kUnit, -off);
      }
    }
  }
  float l_tot[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    l_tot[cg] = l_run[cg];
    l_tot[cg] += shfl_xor_f32(l_tot[cg], 16);
    l_tot[cg] += shfl_xor_f32(l_tot[cg], 32);
  }
  if constexpr (NW > 1 && !kShare) {
    // Waves 1.. publish their (m, l, o) in LDS; wave 0 rescales them to the
    // common max and adds them in wave order (the merge rule of the partition
    // states, inside the workgroup), then writes the item's result.
    __shared__ float sm_m[NW - 1][NCG][16];
    __shared__ float sm_l[NW - 1][NCG][16];
    typedef f32x4 xo_t[NCG][8][64];
    auto xo = [&](int w) __attribute__((always_inline)) -> xo_t& {
      if constexpr (kLdsK && sizeof(xo_t) <= 4 * kSlotBlk) {
        // wave w + 1 publishes its o in its own K slot, which its loop no longer uses
        return *reinterpret_cast<xo_t*>(&k_lds[w + 1][0]);
      } else {
        __shared__ f32x4 sm_o[NW - 1][NCG][8][64];
        return sm_o[w];
      }
    };
    if (wave > 0) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        if (c == 0) {
          sm_m[wave - 1][cg][n] = m_run[cg];
          sm_l[wave - 1][cg][n] = l_tot[cg];
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) xo(wave - 1)[cg][dt][lane] = oacc[cg][dt];
      }
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      float M = m_run[cg];
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) M = fmaxf(M, sm_m[w][cg][n]);
      const float Mu = M == -INFINITY ? 0.f : M;     // no token in the whole item: all weights 0
      const float f0 = __builtin_amdgcn_exp2f(m_run[cg] - Mu);
      float l = l_tot[cg] * f0;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[cg][dt] *= f0;
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm_m[w][cg][n] - Mu);
        l += sm_l[w][cg][n] * f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[cg][dt] += xo(w)[cg][dt][lane] * f;
      }
      m_run[cg] = M;
      l_tot[cg] = l;
    }
  }
  const int64_t slot = ((int64_t)s * a.num_kv_heads + kvh) * a.max_parts + part;
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int v = v0 + 16 * cg + n;
    if (v >= GV) continue;
    if constexpr (kShare && NCG == 2 && M::kBits == 16) {
      if (nparts == 1) {
        // bf16 tile sharing, one partition: the outputs go out through this
        // wave's 8 KiB of a stage (rows of 256 B per pair; 16-byte chunk k of
        // pair p at chunk k ^ (p & 15), so the 16 pairs of a write hit distinct
        // banks), and each lane then stores 16 contiguous bytes, each
        // instruction four whole rows, instead of 8 bytes of 16 rows
        uint8_t* ob = (wave < 4 ? kv_lds0 : kv_lds1) + (wave & 3) * 8192;
        const int p = 16 * cg + n;
        const float inv = l_tot[cg] > 0.f ? a.v_scale / l_tot[cg] : 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          u32x2 w;
          w[0] = uint32_t(f32_to_bf16_bits(oacc[cg][dt][0] * inv)) | (uint32_t(f32_to_bf16_bits(oacc[cg][dt][1] * inv)) << 16);
          w[1] = uint32_t(f32_to_bf16_bits(oacc[cg][dt][2] * inv)) | (uint32_t(f32_to_bf16_bits(oacc[cg][dt][3] * inv)) << 16);
          const int k = 2 * dt + (c >> 1);
          *reinterpret_cast<u32x2*>(ob + p * 256 + ((k ^ (p & 15)) << 4) + ((c & 1) << 3)) = w;
        }
        continue;
      }
    }
    if (nparts == 1) {
      const int qi = v / group;
      const int h = v - qi * group;
      const float inv = l_tot[cg] > 0.f ? a.v_scale / l_tot[cg] : 0.f;
      uint16_t* out = static_cast<uint16_t*>(a.out) +
                      (((int64_t)s * QL + qi) * a.num_heads + (int64_t)kvh * group + h) * kD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        u32x2 w;
        w[0] = uint32_t(f32_to_bf16_bits(oacc[cg][dt][0] * inv)) | (uint32_t(f32_to_bf16_bits(oacc[cg][dt][1] * inv)) << 16);
        w[1] = uint32_t(f32_to_bf16_bits(oacc[cg][dt][2] * inv)) | (uint32_t(f32_to_bf16_bits(oacc[cg][dt][3] * inv)) << 16);
        *reinterpret_cast<u32x2*>(out + 16 * dt + 4 * c) = w;
      }
    } else {
      float* po = a.part_o + (slot * GV + v) * kD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * c) = oacc[cg][dt] * a.v_scale;
      if (c == 0) {
        a.part_m[slot * GV + v] = m_run[cg];
        a.part_l[slot * GV + v] = l_tot[cg];
      }
    }
  }
  if constexpr (kShare && NCG == 2 && M::kBits == 16) {
    static_assert(4 * 8192 <= kStageBytes, "four waves' outputs fit a stage");
    if (nparts == 1) {
      const uint8_t* ob = (wave < 4 ? kv_lds0 : kv_lds1) + (wave & 3) * 8192;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int p = 4 * kk + (lane >> 4), j = lane & 15;
        const uint4 x = *reinterpret_cast<const uint4*>(ob + p * 256 + ((j ^ (p & 15)) << 4));
        const int v = v0 + p;
        if (v < GV) {
          const int qi = v / group;
          const int h = v - qi * group;
          uint16_t* out = static_cast<uint16_t*>(a.out) +
                          (((int64_t)s * QL + qi) * a.num_heads + (int64_t)kvh * group + h) * kD;
          *reinterpret_cast<uint4*>(out + 8 * j) = x;
        }
      }
    }
  }
}

// One column group fits two waves per SIMD (<= 256 registers per lane), so
// one wave's compute overlaps the other's loads, and three with an 8-bit or
// 4-bit cache (<= 168 registers); more groups take one wave.
#define PA_MFMA_KERNEL_ATTRS                                          \
  __global__ __launch_bounds__(64 * NW)                               \
  __attribute__((amdgpu_waves_per_eu(                                 \
      (NCG == 1 && KDT != kBF16) ? 3 : (NCG == 1 || (STAGES > 0 && NCG == 2)) ? 2 : 1, 8)))

// Grid schedule: one workgroup per (KV head, sequence, partition) of the dense grid.
template <int KDT, int NCG, int NW, bool STREAM, bool BSCALE, int STAGES>
PA_MFMA_KERNEL_ATTRS void mfma_partition_kernel(const Args a, int group) {
  const Item it = work_item(a);
  partition_item<KDT, NCG, NW, STREAM, BSCALE, STAGES>(a, group, it.s, it.kvh, it.part, it.qb);
}

// List schedule: workgroup i takes item i of the list the plan kernel built,
// longest first, and workgroups past its end exit at once. Workgroups are
// dispatched in index order, so long items start first and short ones fill
// the end; consecutive (similar) items go to consecutive XCDs.
template <int KDT, int NCG, int NW, bool STREAM, bool BSCALE, int STAGES>
PA_MFMA_KERNEL_ATTRS void mfma_partition_list_kernel(const Args a, int group) {
  const int idx = blockIdx.x;
  if (idx >= *a.queue_len) return;
  const int2 w = a.queue_items[idx];            // unit (s * q_blocks + qb) * Hkv + kvh, partition
  const int sq = w.x / a.num_kv_heads;
  const int s = sq / a.q_blocks;
  partition_item<KDT, NCG, NW, STREAM, BSCALE, STAGES>(a, group, s, w.x - sq * a.num_kv_heads, w.y,
                                                       sq - s * a.q_blocks);
}

}  // namespace

bool mfma_share_tiles(int group, int q_len, int nw) {
  return nw > 1 && group * q_len > 16 * kMaxColumnGroups;
}

int mfma_item_blocks(int group, int q_len, int nw) {
  const int gv = group * q_len;
  if (mfma_share_tiles(group, q_len, nw)) {
    const int per_wave = 16 * kShareGroups;
    return ((gv + per_wave - 1) / per_wave + nw - 1) / nw;
  }
  return (gv + 16 * kMaxColumnGroups - 1) / (16 * kMaxColumnGroups);
}

// Default waves per item when they share tiles: 2 for up to 64 pairs of a KV
// head, else 4 (two workgroups per CU), except with a bf16 cache past 4096
// tokens, where 8 (one workgroup per CU: half the items, so half the K/V
// re-reads) measured 5 % ahead at 32 positions over 32K tokens and 1.5 % at
// 64. On shorter sequences 8 waves measured 2-14 % slower (a few tiles per
// item never fill the pipeline), and with fp8 and int4 caches, whose tiles
// are half or a quarter the bytes, 4 waves tied or won (long-context batch,
// 32 positions: e5m2 even, e4m3 and int4 1.5 % ahead; shared-prefix batch, 32
// and 64 positions: 5.5 % ahead).
int mfma_share_default_waves(int group, int q_len, long long max_len, int kv_dtype) {
  const int blocks = (group * q_len + 16 * kShareGroups - 1) / (16 * kShareGroups);
  if (blocks <= 2) return 2;
  return blocks > 4 && max_len > 4096 && kv_dtype == kBF16 && kShareMaxWaves == 8 ? 8 : 4;
}

// Waves per item: 1 to 4 with one column group; 1 or 2 with two or four
// (the LDS exchange holds (NW - 1) x NCG x 8 KiB). With more than one query
// block the waves share tiles instead: 2, 4 or 8.
bool mfma_waves_supported(int group, int q_len, int nw) {
  const int gv = group * q_len;
  if (gv > 16 * kMaxColumnGroups) return nw == 1 || nw == 2 || nw == 4 || (nw == 8 && kShareMaxWaves == 8);
  return nw == 1 || nw == 2 || ((nw == 3 || nw == 4) && gv <= 16);
}

bool mfma_supported(int q_dtype, int kv_dtype, int head_dim, int group, int block_size, int q_len) {
  return q_dtype == kBF16 && (kv_dtype == kBF16 || kv_dtype == kE5M2 || kv_dtype == kE4M3 || kv_dtype == kI4) &&
         head_dim == kD &&
         block_size == kBlockSize && group >= 1 && q_len >= 1 && q_len <= kMaxQueryLen;
}

namespace {

// Timing events, when given, are attached to the kernel's own dispatch
// (start and end of its execution) instead of being separate stream markers.
struct Timing {
  hipEvent_t start, stop;
};

template <int KDT, int NCG, int NW, bool ST, bool BS, int STG>
void launch_one(const Args& a, int group, dim3 grid, bool queue, hipStream_t stream, Timing tm) {
  auto kern = queue ? mfma_partition_list_kernel<KDT, NCG, NW, ST, BS, STG>
                    : mfma_partition_kernel<KDT, NCG, NW, ST, BS, STG>;
  if (tm.start || tm.stop)
    hipExtLaunchKernelGGL(kern, grid, dim3(64 * NW), 0, stream, tm.start, tm.stop, 0, a, group);
  else
    kern<<<grid, 64 * NW, 0, stream>>>(a, group);
}

template <int KDT, int NCG, int NW, bool ST, int STG = 0>
void launch_scaled(const Args& a, int group, dim3 grid, bool queue, hipStream_t stream, Timing tm) {
  if constexpr (KDT == kBF16) launch_one<KDT, NCG, NW, ST, false, STG>(a, group, grid, queue, stream, tm);
  else if constexpr (KDT == kI4) launch_one<KDT, NCG, NW, ST, true, STG>(a, group, grid, queue, stream, tm);
  else if (a.k_bscale != nullptr) launch_one<KDT, NCG, NW, ST, true, STG>(a, group, grid, queue, stream, tm);
  else launch_one<KDT, NCG, NW, ST, false, STG>(a, group, grid, queue, stream, tm);
}

// LDS stages of the tile-sharing kernels: two of 33 KiB. The copies of the
// next tile land in one stage while the compute reads the other (the compiler
// tells them apart and does not hold the reads for those copies), and the
// barrier before each tile both covers its copies and frees the other stage.
// More stages were measured slower: their LDS takes occupancy and the
// prefetch depth does not pay for it once the copies overlap the compute.
template <int KDT, int NW>
constexpr int share_stages() {
  return 2;
}

template <int KDT>
void launch_kdt(const Args& a, int group, int ncg, int nw, bool share, dim3 grid, bool queue, hipStream_t stream,
                Timing tm) {
  const bool st = a.q_blocks == 1;   // several query blocks: share tiles through the caches
  if (share) {
    constexpr int G = kShareGroups;
    if (nw == 2 && st) launch_scaled<KDT, G, 2, true, share_stages<KDT, 2>()>(a, group, grid, queue, stream, tm);
    else if (nw == 2) launch_scaled<KDT, G, 2, false, share_stages<KDT, 2>()>(a, group, grid, queue, stream, tm);
    else if (nw == 4 && st) launch_scaled<KDT, G, 4, true, share_stages<KDT, 4>()>(a, group, grid, queue, stream, tm);
    else if (nw == 4) launch_scaled<KDT, G, 4, false, share_stages<KDT, 4>()>(a, group, grid, queue, stream, tm);
    else if constexpr (kShareMaxWaves == 8) {
      if (st) launch_scaled<KDT, G, 8, true, share_stages<KDT, 8>()>(a, group, grid, queue, stream, tm);
      else launch_scaled<KDT, G, 8, false, share_stages<KDT, 8>()>(a, group, grid, queue, stream, tm);
    }
  }
  else if (ncg == 1 && nw == 1) launch_scaled<KDT, 1, 1, true>(a, group, grid, queue, stream, tm);
  else if (ncg == 1 && nw == 2) launch_scaled<KDT, 1, 2, true>(a, group, grid, queue, stream, tm);
  else if (ncg == 1 && nw == 3) launch_scaled<KDT, 1, 3, true>(a, group, grid, queue, stream, tm);
  else if (ncg == 1) launch_scaled<KDT, 1, 4, true>(a, group, grid, queue, stream, tm);
  else if (ncg == 2 && nw == 1) launch_scaled<KDT, 2, 1, true>(a, group, grid, queue, stream, tm);
  else if (ncg == 2) launch_scaled<KDT, 2, 2, true>(a, group, grid, queue, stream, tm);
  else if (nw == 1 && st) launch_scaled<KDT, 4, 1, true>(a, group, grid, queue, stream, tm);
  else if (nw == 1) launch_scaled<KDT, 4, 1, false>(a, group, grid, queue, stream, tm);
  else if (st) launch_scaled<KDT, 4, 2, true>(a, group, grid, queue, stream, tm);
  else launch_scaled<KDT, 4, 2, false>(a, group, grid, queue, stream, tm);
}

}  // namespace

hipError_t launch_mfma(const Args& a, int q_dtype, int kv_dtype, int head_dim, int group,
                       hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const Timing tm{ev_start, ev_stop};
  if (!mfma_supported(q_dtype, kv_dtype, head_dim, group, kBlockSize, a.q_len)) return hipErrorInvalidValue;
  const int gv = group * a.q_len;                 // virtual heads per KV head, in blocks of up to 64
  const int ncg = gv <= 16 ? 1 : gv <= 32 ? 2 : 4;
  const int nw = a.waves_per_item;
  if (!mfma_waves_supported(group, a.q_len, nw)) return hipErrorInvalidValue;
  const bool share = mfma_share_tiles(group, a.q_len, nw);
  if (a.q_blocks != mfma_item_blocks(group, a.q_len, nw)) return hipErrorInvalidValue;
  if ((kv_dtype == kI4) != (a.k_bscale != nullptr && a.v_bscale != nullptr) && kv_dtype != kE5M2 &&
      kv_dtype != kE4M3)
    return hipErrorInvalidValue;                  // int4 needs both scale arrays; bf16 takes none
  const bool queue = a.queue_items != nullptr;
  const dim3 grid = queue ? dim3((unsigned)a.queue_workgroups) : partition_grid(a);   // list: one per possible item
  if (kv_dtype == kBF16) launch_kdt<kBF16>(a, group, ncg, nw, share, grid, queue, stream, tm);
  else if (kv_dtype == kE5M2) launch_kdt<kE5M2>(a, group, ncg, nw, share, grid, queue, stream, tm);
  else if (kv_dtype == kE4M3) launch_kdt<kE4M3>(a, group, ncg, nw, share, grid, queue, stream, tm);
  else launch_kdt<kI4>(a, group, ncg, nw, share, grid, queue, stream, tm);
  return hipGetLastError();
}

}  // namespace pa
