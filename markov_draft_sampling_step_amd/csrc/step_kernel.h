#pragma once
// MI355X (gfx950, CDNA4) DSpark sequential Markov draft-sampling step.
//
// One kernel launch per draft step; one 8-wave workgroup per CU. The
// vocabulary is cut into 128-token slabs (four 32-token units, one per
// SIMD); a workgroup owns the slabs blockIdx.x + G i, and the two waves on
// each SIMD take every other one of them, so every SIMD gets the same share
// of the vocabulary. Each wave handles all request rows of its units:
//   * the rows' Markov embeddings w1[prev] sit in LDS (16-byte chunks,
//     XOR-swizzled by row so the MFMA operand reads hit distinct banks);
//   * each wave streams its unit's w2 rows from HBM once per step, straight
//     into v_mfma_f32_16x16x32_bf16 A operands (16-byte loads, issued before
//     anything else at kernel start and again as soon as a unit's last
//     contraction has issued); tokens sit on the MFMA's M side in an order
//     that leaves each lane with 8 consecutive tokens of one row, so the
//     base read and the cache write are 16-byte vectors with no transpose;
//   * the epilogue (bf16 bias, bf16 add, multiplier / soft cap, cache store)
//     and the Gumbel noise run in registers. The noise is bounded, not
//     computed: MurmurHash3 gives h, and a 2050-entry table in LDS, indexed
//     by the exponent and top 6 mantissa bits of float(h), holds an upper
//     bound of the noise over each bucket of h. A lane keeps the largest two
//     bounds of its row; the workgroup takes one exact key (binary64 logs,
//     IEEE division) per row, for the element with the largest bound, and
//     only re-scans a row when another bound reaches that key;
//   * with a soft cap, the output transform is looked up in a host-built
//     table of all 32768 bf16 magnitudes (the transform is odd), copied to
//     LDS address 0;
//   * per-row winners go out as one packed (order-preserving key, ~id)
//     64-bit atomicMax per row per workgroup, into one of 8 slot groups; the
//     next step's kernel decodes the largest (no fences: the kernel boundary
//     orders the steps), and in the last step the workgroup that takes the
//     last device-scope ticket writes the last tokens. One launch per step.
//
// The definition followed is stated in include/markov.h, with the pages it
// comes from (vLLM Markov-drafter API pages: kimi_k3 `_gumbel_key` and the
// module's exactness paragraph; muse_spark cutedsl `_logit`, `_gumbel`,
// `_murmur_prefix`, `_combine`, `_w1_row`, `markov_step`).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "markov.h"

// The launch arguments of every step kernel (shared by the translation units
// of the rank classes, hence outside the anonymous namespace).
namespace markov_impl {
struct StepArgs {
  const uint16_t* base;
  const uint16_t* w1;
  const uint16_t* w2;
  const int64_t* prev;
  const int64_t* seeds;
  const int64_t* positions;
  const float* temperature;
  uint16_t* cache;
  int64_t* tokens;
  unsigned long long* slots;  // [3][SG][rows] packed winners, step s uses s % 3
  unsigned int* ticket;       // workgroups of the last step done so far (zero between calls)
  const float* gtable;        // the noise bound table (in the workspace)
  const uint32_t* ttable;     // the transform table's stamp, then its 32768 entries
  uint16_t* bias_out;
  unsigned long long* winners;  // greedy: [rows, k] packed winners (NULL: not written)
  const uint8_t* w2q;           // E4M3 w2 [V, R] codes (the V_W8 variant)
  const uint16_t* w2s;          // its FP16 row scales [V]
  // vocabulary shard: the step on tokens [id_offset, id_offset + V) of a
  // vocabulary of V_total (w1 has V_total rows), fed from prev[r *
  // feed_stride] at every step; its per-row winner (global id) goes to
  // packets[r] instead of a token (NULL: not a shard)
  unsigned long long* packets;
  int64_t feed_stride;
  int id_offset, V_total;
  int rows, V, R, k, step, nslabs, mode;
  int tt_layout;              // LDS holds the transform table at address 0
  float mult, inv_cap, cap;
  int has_cap;
  float inf;                  // +infinity, opaque to the compiler (see the noise loop)
};

typedef void (*StepFn)(StepArgs);
}  // namespace markov_impl

namespace {

constexpr int NWV = 8;                 // waves per workgroup (two per SIMD)
constexpr int NTH = 64 * NWV;          // threads per workgroup
constexpr int TOK_PER_WAVE = 32;       // two 16-token MFMA M tiles
constexpr int SLAB = 4 * TOK_PER_WAVE; // one unit per SIMD
constexpr int NONE = 0x7fffffff;       // id of "no element yet"
constexpr int ROWS_CAP = NTH;          // the prologue gives every row one thread
constexpr int MRB_MAX = 8;             // row blocks one wave keeps in registers
constexpr int FB_BATCH = 8;            // cache words in flight per lane in a fallback scan
constexpr int WAIT_VM0 = 0x0F70;       // s_waitcnt vmcnt(0), the other counters free (gfx9 encoding)
constexpr size_t LDS_MAX = 160 * 1024;
// Winner slot groups: workgroup b publishes into group b % SG, and a step's
// winner is the largest value over the groups. Device-scope atomics on one
// cache line are served one after another, so SG groups cut the queue on
// each line SG-fold; the reader pays SG loads per row.
constexpr int SG = 8;

enum Mode { MODE_SAMPLE = 0, MODE_SAMPLE_EXACT = 1, MODE_BIAS = 2, MODE_SAMPLE_FALLBACK = 3, MODE_GREEDY = 4 };

// Compile-time variants of the step kernel (bits):
//   V_EXACT   the test-only variant that takes the exact key of every element;
//   V_GREEDY  every row at temperature 0: no noise table, no hashing, an
//             exact in-register argmax under the total order (NaN and -inf
//             included, so no re-scan and the cache write may be skipped).
//   V_W8      w2 as E4M3 codes with an FP16 scale per row (the Edge-LLM
//             page's `dsparkMarkovGreedyFusedStepFp8` layout): the codes are
//             decoded to bf16 (exact: every E4M3 value is a bf16) for the
//             same MFMA contraction, and the fp32 sum is scaled before it is
//             rounded to bf16.
constexpr int V_SAMPLE = 0, V_EXACT = 1, V_GREEDY = 2, V_W8 = 4;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

using markov_impl::StepArgs;
using markov_impl::StepFn;

// ---------------------------------------------------------------- numbers

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two binary32 -> one word of two bf16 (round to nearest even; one
// hardware v_cvt_pk_bf16_f32), `a` in the low half.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// ---------------------------------------------------------------- noise hash
// MurmurHash3_x86_32 over the 16-byte message (lo32 S, hi32 S, lo32 P, id),
// seed 0, S = seed ^ (step << 32), P = position - 1 + 2^30. The three
// per-row words are folded once per row (`row_prefix`); the id word's
// scramble depends on the token only and is shared by all rows.
constexpr uint32_t MM_C1 = 0xcc9e2d51u, MM_C2 = 0x1b873593u;

__device__ __forceinline__ uint32_t rotl32(uint32_t x, int r) { return (x << r) | (x >> (32 - r)); }

__device__ __forceinline__ uint32_t mm_block(uint32_t h, uint32_t k) {
  k *= MM_C1;
  k = rotl32(k, 15);
  k *= MM_C2;
  h ^= k;
  h = rotl32(h, 13);
  return h * 5u + 0xe6546b64u;
}

__device__ __forceinline__ uint32_t mm_token_word(uint32_t id) {
  uint32_t k = id * MM_C1;
  k = rotl32(k, 15);
  return k * MM_C2;
}

// h * 5 + c as a shift-add and an add (two full-rate ops; left to itself
// the compiler picks a 64-bit multiply-add)
__device__ __forceinline__ uint32_t times5_plus(uint32_t h, uint32_t c) {
  uint32_t r;
  asm("v_lshl_add_u32 %0, %1, 2, %1" : "=v"(r) : "v"(h));
  return r + c;
}

// The last block and the finaliser, from the row prefix and the token word
// both already rotated left by 13 (rotation distributes over xor, so the
// block's rotation moves onto the two operands: once per row, and once per
// token for all rows).
__device__ __forceinline__ uint32_t mm_finish_rot(uint32_t prefix_rot, uint32_t token_word_rot) {
  uint32_t h = prefix_rot ^ token_word_rot;
  h = times5_plus(h, 0xe6546b64u);
  h ^= 16u;                       // message length in bytes
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

__device__ __forceinline__ uint32_t mm_finish(uint32_t prefix, uint32_t token_word) {
  return mm_finish_rot(rotl32(prefix, 13), rotl32(token_word, 13));
}

__device__ __forceinline__ uint32_t row_prefix_of(int64_t seed, int step, int64_t position) {
  uint64_t S = (uint64_t)seed ^ ((uint64_t)(uint32_t)step << 32);
  int64_t P = position - 1 + ((int64_t)1 << 30);
  uint32_t h = mm_block(0u, (uint32_t)S);
  h = mm_block(h, (uint32_t)(S >> 32));
  return mm_block(h, (uint32_t)(uint64_t)P);
}

// u = RN32((h + 1/2) 2^-32): (lo16 + 1/2) 2^-32 is exact, and one fma adds
// hi16 * 2^-16 with the only rounding.
__host__ __device__ __forceinline__ float uniform_of(uint32_t h) {
  float hi = (float)(h >> 16), lo = (float)(h & 0xffffu);
  return __builtin_fmaf(hi, 0x1p-16f, __builtin_fmaf(lo, 0x1p-32f, 0x1p-33f));
}

// ---------------------------------------------------------------- keys
// Exact key: RN32(RN32(l / T) - lb), lb = RN32(log(-L)), L = log(1 - u) in
// the pages' stable form (a Horner series below u = 1/4, else a log of
// max(1 - u, 2^-24)). Logs are taken in binary64 and rounded once.
__host__ __device__ __forceinline__ float log1m_exact(float u) {
  if (u < 0.25f) {
    float p = 0.125f;
    p = __builtin_fmaf(u, p, 1.0f / 7.0f);
    p = __builtin_fmaf(u, p, 1.0f / 6.0f);
    p = __builtin_fmaf(u, p, 1.0f / 5.0f);
    p = __builtin_fmaf(u, p, 0.25f);
    p = __builtin_fmaf(u, p, 1.0f / 3.0f);
    p = __builtin_fmaf(u, p, 0.5f);
    p = __builtin_fmaf(u, p, 1.0f);
    return p * (-u);
  }
  float x = fmaxf(1.0f - u, 0x1p-24f);
  return (float)log((double)x);
}

__host__ __device__ __forceinline__ float noise_lb(uint32_t h) {
  const float L = log1m_exact(uniform_of(h));
  return (float)log((double)(-L));
}

// key_exact(l, T, h) is NaN exactly for these (its noise term is finite)
__device__ __forceinline__ bool key_is_nan(float l, float T) {
  return __builtin_isnan(l) || __builtin_isnan(T) || (__builtin_isinf(l) && __builtin_isinf(T));
}

__device__ __forceinline__ float key_exact(float l, float T, uint32_t h) {
  const float lb = noise_lb(h);
  float q = l / T;
  return q - lb;
}

// Noise bound table. Bucket b of h: b = 0 for h = 0, else
// (bits(float(h)) >> 17) - 8127, i.e. the exponent and the top 6 mantissa
// bits of the nearest binary32 to h (1 .. 2049; 2049 is h rounding to
// 2^32). gtable[b] = (A, B) is a line in float(h) on or above the noise -lb
// of every h in the bucket: RN32(fma(B, float(h), A)) >= -lb(h). The host
// builds it from the chord of the noise over the bucket and lifts it by the
// largest shortfall found on a grid of the bucket, plus 1e-5 (the noise and
// the line both fall as h grows, so a shortfall between two grid points is
// at most the line at the next point below the noise at this one). The
// kernel's upper bound of an exact key is then
//   hi = fma(l, RN(1/T), fma(B, float(h), A)),  up = fma(|hi|, 2^-19, hi)
// (2^-19 |hi| covers the roundings of l / T, of the key and of hi, and the
// 3-bit id the kernel packs into up's low bits). A second table holds a
// constant bound per bucket, the largest noise on the bucket's grid plus
// 1e-5 (the noise at its first h, as the noise falls with h): the plans with
// two row groups use it, as the line's float(h) operand would cost them
// registers they lack.
constexpr int GT_BASE = 8127;
constexpr int GT_N = 2050;
constexpr int GT_PAD = 2176;               // stored pairs: 17 chunks of 1 KiB
constexpr uint32_t GT_BYTES = GT_PAD * 8;
constexpr int GTC_PAD = 2112;              // stored constants: 8.25 chunks of 1 KiB
constexpr uint32_t GTC_BYTES = GTC_PAD * 4;
constexpr uint32_t TABLES_BYTES = GT_BYTES + GTC_BYTES;   // both, at the workspace's start
constexpr int GT_GRID = 1024;              // grid intervals per bucket in the host's check

// Transform table. The output transform maps a bf16 x (the bf16 sum of base
// and bias) to the cached bf16 c, and every step of it (the multiplier, the
// scaling by RN(1/cap), tanh, the scaling by cap, the roundings) is odd, so
// c(-x) = -c(x) bit for bit and the map is a table over the 32768 values of
// |x|. The host fills it with correctly rounded arithmetic for one (mult,
// cap) and stamps it with both; a kernel whose own (mult, cap) match the
// stamp looks c up in LDS (two reads per word of two values, the sign put
// back with one xor), else it evaluates the transform itself.
constexpr uint32_t TT_MAGIC = 0x4d545431u;
constexpr uint32_t TT_HEAD = 256;          // stamp: magic, bits(mult), bits(cap), then zeros
constexpr uint32_t TT_BYTES = 65536;       // 32768 bf16 entries, index |x|
constexpr uint32_t WS_TT = TABLES_BYTES;   // workspace offset of the stamp
constexpr uint32_t WS_TICKET = WS_TT + TT_HEAD + TT_BYTES;  // the last step's completion count
constexpr uint32_t WS_SLOTS = WS_TICKET + 256;              // the slot arrays follow

__device__ __forceinline__ uint32_t gt_index(float fh) {
  return __builtin_elementwise_sub_sat(__float_as_uint(fh) >> 17, (uint32_t)GT_BASE);
}

// the table's bound of the noise -lb(h): the line (LIN) or the constant
template <bool LIN>
__device__ __forceinline__ float noise_bound(const void* tab, uint32_t h) {
  const float fh = (float)h;
  if (LIN) {
    const float2 ab = ((const float2*)tab)[gt_index(fh)];
    return __builtin_fmaf(ab.y, fh, ab.x);
  }
  return ((const float*)tab)[gt_index(fh)];
}

__device__ __forceinline__ float key_upper(float l, float rcpT, float gh) {
  const float hi = __builtin_fmaf(l, rcpT, gh);
  return __builtin_fmaf(fabsf(hi), 0x1p-19f, hi);
}

// The slot loop keeps, per row, the largest estimates fma(l, RN(1/T), bound)
// with the element's index in the low 3 bits, without key_upper's margin;
// the margin, monotone in the estimate, is added to the kept value once.
// 2^-18 |v| is at least 32 of v's ulps: the 2^-19 of key_upper plus the
// packed bits and an estimate a binade above v.
__device__ __forceinline__ float slack_up(float v) { return __builtin_fmaf(fabsf(v), 0x1p-18f, v); }

// The total order of every argmax here: a NaN beats every non-NaN, lower
// id among NaNs; otherwise the larger value, and equal values (so -0 == +0)
// go to the lower id.
__device__ __forceinline__ bool before(float v1, int i1, float v2, int i2) {
  bool n1 = __builtin_isnan(v1), n2 = __builtin_isnan(v2);
  return (v1 > v2) || (v1 == v2 && i1 < i2) || (n1 && (!n2 || i1 < i2));
}

// Order-preserving 64-bit image of (key, id) under that order: the high word
// maps every NaN to the top and -0 to +0; the low word is ~id, so the lower
// id of equal keys is the larger word. Zero is below every real element.
__device__ __forceinline__ unsigned long long pack_winner(float v, int id) {
  uint32_t o;
  if (__builtin_isnan(v)) {
    o = 0xffffffffu;
  } else {
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0u;
    o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  return ((unsigned long long)o << 32) | (unsigned long long)(uint32_t)(~(uint32_t)id);
}

// The order key of a value (the high word of pack_winner), and back: every
// NaN decodes to a NaN, -0 to +0.
__device__ __forceinline__ uint32_t order_key(float v) { return (uint32_t)(pack_winner(v, 0) >> 32); }
__device__ __forceinline__ float order_value(uint32_t o) {
  return o == 0xffffffffu ? __builtin_nanf("") : __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// The winner slot of a row decodes to its token id.
__device__ __forceinline__ int64_t slot_token(unsigned long long w) {
  return (int64_t)(uint32_t)(~(uint32_t)w);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Workgroup barrier for LDS data only: this wave's LDS operations are
// complete, then all waves meet. (__syncthreads also waits for every
// outstanding global load, which would hold the prologue up on the w2 tiles
// already in flight.) The asm keeps the compiler from moving memory
// operations across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N vector memory operations of this wave are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// A cache word written by another wave of this workgroup (agent-coherent load).
__device__ __forceinline__ uint32_t load_cache_word(const uint16_t* cache, size_t elem_even) {
  return __hip_atomic_load((const uint32_t*)(cache + elem_even), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- output transform
// tanh for the soft cap: below |z| = 0.625 an odd polynomial z + z^3 P(z^2),
// P of degree 5 in z^2 (the Taylor series' odd terms through z^13, each
// coefficient adjusted by a fit to tanh on that interval and rounded to
// binary32); this binary32 Horner evaluation is within 0.73 ulp of tanh over
// every binary32 z in [2^-8, 0.625] (a CPU sweep, its worst case confirmed in
// 50-digit arithmetic). Above, 1 - 2 / (e^{2|z|} + 1) with the hardware exp2
// and reciprocal (about 2 ulp). The cache rounds the result to bf16.
__device__ __forceinline__ float tanh_poly(float z) {
  const float t = z * z;
  float p = 0x1.18dc88p-9f;
  p = __builtin_fmaf(p, t, -0x1.0bf272p-7f);
  p = __builtin_fmaf(p, t, 0x1.638a82p-6f);
  p = __builtin_fmaf(p, t, -0x1.b9ee7p-5f);
  p = __builtin_fmaf(p, t, 0x1.111066p-3f);
  p = __builtin_fmaf(p, t, -0x1.555554p-2f);
  return __builtin_fmaf(t * z, p, z);
}

__device__ __forceinline__ float tanh_fast(float z) {
  const float az = fabsf(z);
  const float e = __builtin_amdgcn_exp2f(az * 2.88539008177792681f);
  const float r = __builtin_amdgcn_rcpf(e + 1.0f);
  const float yl = __builtin_copysignf(__builtin_fmaf(-2.0f, r, 1.0f), z);
  return az < 0.625f ? tanh_poly(z) : yl;
}

// c of both bf16 values of word x from the transform table at LDS address
// 0: entry |x| sits at byte 2 |x|, which one SDWA shift forms from either
// half of x (the sign bit falls out of the 16-bit result).
__device__ __forceinline__ uint32_t tt_addr_lo(uint32_t x) {
  uint32_t r;
  asm("v_lshlrev_b16_sdwa %0, 1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_0"
      : "=v"(r) : "v"(x));
  return r;
}

__device__ __forceinline__ uint32_t tt_addr_hi(uint32_t x) {
  uint32_t r;
  asm("v_lshlrev_b16_sdwa %0, 1, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
      : "=v"(r) : "v"(x));
  return r;
}

typedef __attribute__((address_space(3))) const uint16_t lds_u16_t;

__device__ __forceinline__ uint32_t tt_map(uint32_t x) {
  const uint32_t lo = *(lds_u16_t*)(size_t)tt_addr_lo(x);
  const uint32_t hi = *(lds_u16_t*)(size_t)tt_addr_hi(x);
  return (lo | (hi << 16)) ^ (x & 0x80008000u);
}

// ---------------------------------------------------------------- tiles

// The w2 rows of one 32-token unit as MFMA A operands: lane (g, m) holds
// k-chunks 4i + g of tokens t0 = tok0 + 8 (m >> 2) + (m & 3) (A0) and t0 + 4
// (A1); tokens past the vocabulary read its last row (never stored).
// Ordinary (not nontemporal) loads: the table is read again by the next
// step, and unmarked lines of it stay in the memory-side cache between steps
// (measured: a nontemporal tile stream made the step about 5% slower).
template <int KB>
__device__ __forceinline__ void load_w2_tile(const uint16_t* w2, int V, int R, int tok0, int m, int g,
                                             bool kzero, bf16x8_t* A0, bf16x8_t* A1) {
  const int t0 = tok0 + 8 * (m >> 2) + (m & 3);
  const int ta = t0 < V ? t0 : V - 1, tb = t0 + 4 < V ? t0 + 4 : V - 1;
  const uint16_t* pa = w2 + (size_t)ta * R;
  const uint16_t* pb = w2 + (size_t)tb * R;
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    if (kzero) {
      A0[i] = (bf16x8_t){};
      A1[i] = (bf16x8_t){};
    } else {
      const int ch = 4 * i + g;
      A0[i] = *(const bf16x8_t*)(pa + ch * 8);
      A1[i] = *(const bf16x8_t*)(pb + ch * 8);
    }
  }
}

// The k-chunk (8 consecutive elements) that lane group g feeds to MFMA i. With
// bf16 w2, chunk 4i + g (one 16-byte load per chunk). With E4M3 w2 a 16-byte
// load holds two chunks, so lane group g takes chunks 8 (i / 2) + 2g and the
// next for MFMAs i = 2p, 2p + 1 (the sum over k is the same in any order, and
// the embedding operand reads the same chunks).
template <int KB, bool W8>
__device__ __forceinline__ int chunk_of(int i, int g) {
  return (W8 && KB >= 2) ? 8 * (i >> 1) + 2 * g + (i & 1) : 4 * i + g;
}

// The E4M3 codes of one 32-token unit, raw (decoded by decode_w2q_tile once
// they are needed): lane (g, m) loads, for tokens t0 and t0 + 4 as in
// load_w2_tile, 16 bytes (two chunks) per pair of MFMAs, or with KB = 1 the 8
// bytes of chunk g; and the FP16 scales of the 8 tokens tok0 + 8g .. +7 whose
// bias it finishes (one 16-byte load; none past the vocabulary).
template <int KB>
__device__ __forceinline__ void load_w2q_tile(const uint8_t* q, const uint16_t* sc, int V, int R,
                                              int tok0, int m, int g, bool kzero, u32x4_t* Qa,
                                              u32x4_t* Qb, u32x4_t& S) {
  constexpr int KP = KB >= 2 ? KB / 2 : 1;
  const int t0 = tok0 + 8 * (m >> 2) + (m & 3);
  const int ta = t0 < V ? t0 : V - 1, tb = t0 + 4 < V ? t0 + 4 : V - 1;
  const uint8_t* pa = q + (size_t)ta * R;
  const uint8_t* pb = q + (size_t)tb * R;
  if (KB == 1) {
    if (kzero) {
      Qa[0] = (u32x4_t){0u, 0u, 0u, 0u};
      Qb[0] = (u32x4_t){0u, 0u, 0u, 0u};
    } else {
      const uint2 x = *(const uint2*)(pa + g * 8), y = *(const uint2*)(pb + g * 8);
      Qa[0] = (u32x4_t){x.x, x.y, 0u, 0u};
      Qb[0] = (u32x4_t){y.x, y.y, 0u, 0u};
    }
  } else {
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      Qa[p] = *(const u32x4_t*)(pa + 64 * p + 16 * g);
      Qb[p] = *(const u32x4_t*)(pb + 64 * p + 16 * g);
    }
  }
  const int tg = tok0 + 8 * g;
  S = (u32x4_t){0u, 0u, 0u, 0u};
  if (tg < V) S = *(const u32x4_t*)(sc + tg);
}

// 8 E4M3 codes (bytes of lo, then of hi) to 8 bf16, in order: two codes per
// v_cvt_scalef32_pk_bf16_fp8 at scale 1.
__device__ __forceinline__ bf16x8_t decode8(uint32_t lo, uint32_t hi) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return (bf16x8_t){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The binary16 halves of a word as binary32 (exact). Each half goes through a
// scalar _Float16: a bit cast of a whole word to a two-element _Float16
// vector, taken from an element of a wider vector, was compiled here into
// conversions of the first element only.
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

template <int KB>
__device__ __forceinline__ void decode_w2q_tile(const u32x4_t* Qa, const u32x4_t* Qb, bf16x8_t* A0,
                                                bf16x8_t* A1) {
  if (KB == 1) {
    A0[0] = decode8(Qa[0].x, Qa[0].y);
    A1[0] = decode8(Qb[0].x, Qb[0].y);
  } else {
#pragma unroll
    for (int p = 0; p < KB / 2; ++p) {
      A0[2 * p] = decode8(Qa[p].x, Qa[p].y);
      A0[2 * p + 1] = decode8(Qa[p].z, Qa[p].w);
      A1[2 * p] = decode8(Qb[p].x, Qb[p].y);
      A1[2 * p + 1] = decode8(Qb[p].z, Qb[p].w);
    }
  }
}

// The bias of one 16-row block for the wave's 32 tokens: lane (g, m) gets
// row n = n0 + m (n0 = 16 rb), tokens tg .. tg+3 in c0 and tg+4 .. tg+7 in
// c1. The swizzle mask is below 16, so n & swz = m & swz: the lane's part of
// the address is the same for every block.
template <int KB, bool W8 = false>
__device__ __forceinline__ void block_bias(const bf16x8_t* A0, const bf16x8_t* A1, const uint16_t* emb,
                                           int n0, int m, int R, int g, int swz, bool kzero, f32x4_t& c0,
                                           f32x4_t& c1) {
  c0 = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  c1 = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    bf16x8_t B;
    if (kzero) {
      B = (bf16x8_t){};
    } else {
      const int ch = chunk_of<KB, W8>(i, g);
      B = *(const bf16x8_t*)(emb + (size_t)n0 * R + (m * R + ((ch ^ (m & swz)) * 8)));
    }
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[i], B, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[i], B, c1, 0, 0, 0);
  }
}

// Per LDS row n, one 16-byte record: rk = row * k + step (the row's slice of
// base / cache starts at rk * V), 1/T, the hash prefix and T.
struct RowInfo {
  int rk;
  float rcp;
  uint32_t prefix;
  float T;
};

// v_pk_max_u16: the larger of each 16-bit half
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_u16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// The rows' states after the slab loop. ORDER rows (T = 0, and every row of
// the exact variant): the (key, id) first under the total order. TOP2 rows:
// (v1, id) is the element with the largest upper bound v1, v2 the largest
// upper bound among all other elements, l the logit of element id (so its
// exact key needs no read of the cache). sp: some element had a non-finite
// estimate (noisy rows) or a NaN / -inf logit (T = 0 rows). A workgroup
// accumulates them per row in LDS with atomics: the winner as the packed
// order key of (v1, id) (ds_max_u64: a NaN first, then the larger value, the
// lower id on equal values), then, once the winner is known, v2 as the
// order key of every other state's v1 and every state's v2 (ds_max_u32), l
// from the winning lane and sp as ors into one word (l's bf16 bits high, sp
// bit 0).
//
// LDS, all of it dynamic (the kernel declares no static LDS, so the dynamic
// array starts at address 0):
//   [tt]            with the transform-table layout, its 32768 entries (64 KiB)
//                   at address 0, else nothing
//   table           the noise bound table (lines or constants)
//   region0         embeddings [rp][R] bf16
//   info [rp] RowInfo, n_row [rp], n_src [rp], fb_row [rp], fb_thr [rp],
//   misc [64] (per-wave row counts, fallback count, last-workgroup flag),
//   the row accumulators win [rp] u64 and l|sp [rp] u32 (the accumulated v2
//   reuses n_src, free once the embeddings are gathered)
__host__ __device__ __forceinline__ size_t region0_bytes(int rp, int R) { return (size_t)rp * R * 2; }

__host__ __device__ __forceinline__ size_t lds_dynamic(int rp, int R) {
  return region0_bytes(rp, R) + (size_t)rp * 16 + (size_t)rp * 16 + 64 * 4 + (size_t)rp * 12;
}

// the noise table in LDS: the lines for one row group (up to MRB_MAX row
// blocks), the constants for two
__host__ __device__ __forceinline__ size_t lds_table(int rp, bool greedy = false) {
  return greedy ? 0 : (rp >> 4) > MRB_MAX ? GTC_BYTES : GT_BYTES;
}

__host__ __device__ __forceinline__ size_t lds_total(int rp, int R, bool greedy = false) {
  return lds_table(rp, greedy) + lds_dynamic(rp, R);
}

// the transform-table layout: one row group (the lines), a soft cap, and room
__host__ __device__ __forceinline__ bool tt_fits(int rp, int R, bool greedy = false) {
  return (rp >> 4) <= MRB_MAX && TT_BYTES + lds_total(rp, R, greedy) <= LDS_MAX;
}

// ---------------------------------------------------------------- the step
//
// KB = R / 32 (1 for R = 16 with half the chunks zero), RG row groups (1,
// or 2 for more than 8 row blocks: then the two waves of a SIMD split the
// rows, both take every slab of the workgroup and read its w2 tiles through
// L2), MRB = row blocks per wave (a power of two, the wave's real count may
// be lower), VAR = the variant bits (V_EXACT, V_GREEDY). One launch runs
// step a.step.
template <int KB, int RG, int MRB, int VAR>
__global__ __launch_bounds__(NTH) void markov_step_kernel(StepArgs a) {
  constexpr bool EXACT = (VAR & V_EXACT) != 0;
  constexpr bool GREEDY = (VAR & V_GREEDY) != 0;
  constexpr bool W8 = (VAR & V_W8) != 0;
  constexpr int NB = MRB == 1 ? 2 : 1;                   // w2 tiles in flight per wave
  // row blocks contracted ahead (measured: with 4 bf16 blocks, 2 ahead beat 3
  // and 1; the E4M3 plan keeps 3, as with 2 it needs more than 256 registers)
  constexpr int D = (MRB == 4 && !W8) ? 2 : MRB - 1 < 3 ? MRB - 1 : 3;
  constexpr int S = RG == 1 ? 2 : 1;                     // waves splitting one SIMD's slabs
  constexpr bool ROWREG = MRB <= 4;                      // row constants in registers
  constexpr bool LIN = RG == 1;                          // the line bound (else the constant)
  // lanes carry their top element's cached logit (one word per row block;
  // the two-row-group plans have no registers to spare and read it back)
  constexpr bool CARRY = RG == 1;
  constexpr uint32_t TB = GREEDY ? 0u : LIN ? GT_BYTES : GTC_BYTES;   // the table this plan copies to LDS
  extern __shared__ __align__(16) unsigned char lds[];
  // the transform table sits at LDS address 0 only if the dynamic array
  // starts there (no static LDS); its lookups form absolute addresses
  const bool tt_lay = LIN && a.tt_layout != 0 &&
                      (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)lds == 0u;
  const uint32_t tt_off = tt_lay ? TT_BYTES : 0u;
  float* const gtabf = (float*)(lds + tt_off);           // LIN: (A, B) pairs; else constants
  float2* const gtab = (float2*)gtabf;
  const int mode = a.mode;
  const bool bias_mode = mode == MODE_BIAS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tw = wave & 3;
  const int sub = RG == 1 ? wave >> 2 : 0;
  const int wr = RG == 1 ? 0 : wave >> 2;
  const int g = lane >> 4, m = lane & 15;
  const int R = KB >= 2 ? 32 * KB : a.R;
  const int rows = a.rows, rp = (rows + 15) & ~15, V = a.V, K = a.k;
  const int s = a.step;
  const bool shard = a.packets != nullptr;             // uniform
  const int sset = shard ? 0 : s % 3;                  // this launch's slot set
  const bool feed_prev = bias_mode || shard || s == 0; // the feeding token comes from prev
  const int gofs = a.id_offset;                        // global id of local token 0
  const int nslabs = a.nslabs, G = gridDim.x;
  const int cpr = R >> 3;
  const int swz = (cpr < 16 ? cpr : 16) - 1;
  const int nrb = rp >> 4;
  const int my_nrb = nrb > wr ? (nrb - wr + RG - 1) / RG : 0;
  const int slab_step = G * S;
  const int slab0 = blockIdx.x + G * sub;
  const bool kzero = (KB == 1) && (R == 16) && (g >= 2);
  // this wave's units per step: slabs slab0 + i slab_step whose 32 tokens
  // start inside the vocabulary
  int lim = (V - tw * TOK_PER_WAVE + SLAB - 1) / SLAB;
  lim = lim < nslabs ? lim : nslabs;
  const int U = (my_nrb > 0 && slab0 < lim) ? (lim - slab0 + slab_step - 1) / slab_step : 0;


  uint16_t* emb = (uint16_t*)(lds + tt_off + TB);
  const size_t r0 = region0_bytes(rp, R);
  RowInfo* n_info = (RowInfo*)((unsigned char*)emb + r0);
  int* n_row = (int*)(n_info + rp);
  int* n_src = n_row + rp;
  int* fb_row = n_src + rp;
  float* fb_thr = (float*)(fb_row + rp);
  int* misc = (int*)(fb_thr + rp);
  unsigned long long* acc_win = (unsigned long long*)(misc + 64);   // the row accumulators
  uint32_t* acc_lsp = (uint32_t*)(acc_win + rp);
  uint32_t* acc_v2 = (uint32_t*)n_src;                              // once the gather is done

  // 0. this thread's request row: everything the first step needs, in one
  //    round trip
  const int r = tid;
  const bool valid = r < rows;
  float T = 0.0f;
  int64_t tok = 0, seed = 0, pos = 0;
  unsigned long long slot_in[SG];
#pragma unroll
  for (int q = 0; q < SG; ++q) slot_in[q] = 0ull;
  if (valid) {
    // the feeding token: prev at step 0, else the previous step's winner
    // slots (decoded after the wait below). prev is read first and at every
    // step (the caller's array is always there): requested under the step-0
    // branch after the loads below, its 64-bit address arithmetic took a
    // register of a load in flight and waited for it.
    tok = a.prev[(int64_t)r * a.feed_stride];
    if (!bias_mode && !GREEDY) {
      T = a.temperature[r];
      seed = a.seeds[r];
      pos = a.positions[(int64_t)r * K + s];
    }
    if (!feed_prev) {
      const unsigned long long* sp0 = a.slots + (size_t)((s + 2) % 3) * SG * rows + r;
#pragma unroll
      for (int q = 0; q < SG; ++q) slot_in[q] = sp0[(size_t)q * rows];
    }
  }
  // the transform table's stamp (the three words that say whether the table
  // serves this launch's (mult, cap)), with the row data: read later, its
  // loads would wait behind the first tile and the table copies, and so
  // would the base logits and the gather requested after them
  uint32_t tts0 = 0u, tts1 = 0u, tts2 = 0u;
  if (LIN && a.tt_layout != 0) {
    tts0 = a.ttable[0];
    tts1 = a.ttable[1];
    tts2 = a.ttable[2];
  }
  // the row data, waited for before the table copy is issued: a wait the
  // compiler sees, so that no later use of a row register waits for the copy;
  // the empty asm keeps every use of the four values (the row hash) below it,
  // so that all four loads are issued before the one wait
  __builtin_amdgcn_s_waitcnt(WAIT_VM0);
  asm volatile("" : "+v"(T), "+v"(seed), "+v"(pos), "+v"(tok));
  asm volatile("" : "+v"(slot_in[0]), "+v"(slot_in[1]), "+v"(slot_in[2]), "+v"(slot_in[3]),
               "+v"(slot_in[4]), "+v"(slot_in[5]), "+v"(slot_in[6]), "+v"(slot_in[7]));
  asm volatile("" : "+v"(tts0), "+v"(tts1), "+v"(tts2));
  static_assert(SG == 8, "the asm above pins SG slot values");
  // the noise bound table, straight into LDS: waited for with the first tile
  // (before the unit loop), in flight through the row set-up
  if (!bias_mode && !GREEDY) {
    for (int j = wave; j * 64 * 16 < (int)TB; j += NWV) {
      const int p = j * 64 + lane;
      if (p * 16 < (int)TB)
        __builtin_amdgcn_global_load_lds((const void*)((const unsigned char*)a.gtable + (LIN ? 0 : GT_BYTES) +
                                                       (size_t)p * 16),
                                         (__attribute__((address_space(3))) void*)(gtabf + (size_t)j * 256),
                                         16, 0, 0);
    }
  }
  // the transform table likewise (the host asks for this layout only with a
  // soft cap; whether the stamp matches is checked where it is used): its
  // lines come from L2 once one workgroup of an XCD has read them, so it
  // lands well before the first tiles it is waited for with (issued after
  // the gather instead, the Large step took 0.4 us longer)
  if (tt_lay) {
    const unsigned char* src = (const unsigned char*)a.ttable + TT_HEAD;
    for (int j = wave; j * 64 * 16 < (int)TT_BYTES; j += NWV)
      __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)(j * 64 + lane) * 16),
                                       (__attribute__((address_space(3))) void*)(lds + (size_t)j * 1024),
                                       16, 0, 0);
  }
  // everything the row set-up needs from the row data, before the tile loads
  // below
  const bool noisy_r = valid && !bias_mode && !(T == 0.0f);
  const uint64_t bn = __ballot(noisy_r), bz = __ballot(valid && !noisy_r);
  const float rcp_r = 1.0f / T;
  const uint32_t prefix_r = (valid && !bias_mode && !GREEDY) ? row_prefix_of(seed, s, pos) : 0u;
  unsigned long long win_in = 0ull;   // the previous step's packed winner of this row
  if (!feed_prev) {
    win_in = slot_in[0];
#pragma unroll
    for (int q = 1; q < SG; ++q) win_in = slot_in[q] > win_in ? slot_in[q] : win_in;
    tok = slot_token(win_in);
  }
  const int tok32 = (int)tok;
  __builtin_amdgcn_sched_barrier(0);

  // 1. the wave's first w2 tile: it depends on nothing above, and stays in
  //    flight through the row set-up (a wave without units reads clamped
  //    rows). With one row group, only the first wave of each SIMD (the one
  //    with more units) requests it here; the second requests its own after
  //    the embedding gather, so that the gather waits behind half the bytes.
  // (E4M3 tiles are half the bytes: every wave requests its own early, which
  // measured faster there)
  const bool tile_first = RG == 2 || sub == 0 || W8;   // uniform per wave
  // bf16 w2: NB tiles of MFMA operands in flight. E4M3 w2: NB raw tiles in
  // flight (codes and scales) and one decoded tile of operands.
  constexpr int NA = W8 ? 1 : NB;
  constexpr int KP = W8 ? (KB >= 2 ? KB / 2 : 1) : 1;
  bf16x8_t A0[NA][KB], A1[NA][KB];
  u32x4_t Qa[W8 ? NB : 1][KP], Qb[W8 ? NB : 1][KP], QS[W8 ? NB : 1];
  // the tile of the unit at token tok0 into buffer b
  auto tile = [&](int b, int tok0) {
    if constexpr (W8)
      load_w2q_tile<KB>(a.w2q, a.w2s, V, R, tok0, m, g, kzero, Qa[b], Qb[b], QS[b]);
    else
      load_w2_tile<KB>(a.w2, V, R, tok0, m, g, kzero, A0[b], A1[b]);
  };
  if (tile_first) tile(0, (U > 0 ? slab0 : 0) * SLAB + tw * TOK_PER_WAVE);
  __builtin_amdgcn_sched_barrier(0);

  // 2. rows: noisy rows first, so that 16-row blocks are of one kind
  if (lane == 0) {
    misc[wave] = __builtin_popcountll(bn);
    misc[8 + wave] = __builtin_popcountll(bz);
  }
  if (tid == 0) misc[16] = 0;
  lds_barrier();
  {
    int pre_n = 0, pre_z = 0, tot_n = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const int cn = misc[w], cz = misc[8 + w];
      tot_n += cn;
      if (w < wave) {
        pre_n += cn;
        pre_z += cz;
      }
    }
    if (valid) {
      const int pos_n = bias_mode ? r
                      : noisy_r ? pre_n + (int)lanes_below(bn)
                                : tot_n + pre_z + (int)lanes_below(bz);
      n_row[pos_n] = r;
      // the feeding token (any int64 at step 0, clamped as unsigned)
      const uint64_t ut = (uint64_t)tok, last = (uint64_t)(a.V_total - 1);
      n_src[pos_n] = (int)(ut < last ? ut : last);
      n_info[pos_n] = RowInfo{r * K + s, rcp_r, prefix_r, T};
      if (!bias_mode && !shard && blockIdx.x == 0) {
        if (s > 0) {                                                 // previous step's
          a.tokens[(int64_t)r * K + s - 1] = (int64_t)(uint32_t)tok32;
          if (a.winners) a.winners[(int64_t)r * K + s - 1] = win_in;
        }
#pragma unroll
        for (int q = 0; q < SG; ++q)                                  // next step's slots start empty
          a.slots[((size_t)((s + 1) % 3) * SG + q) * rows + r] = 0ull;
      }
    } else if (r < rp) {
      n_row[r] = 0;
      n_src[r] = 0;
      n_info[r] = RowInfo{0, 0.0f, 0u, 0.0f};
    }
    if (r < rp) {   // the row accumulators start empty (v2 below, after the gather)
      acc_win[r] = 0ull;
      acc_lsp[r] = 0u;
    }
  }

  u32x4_t bq[MRB];
  RowInfo ri[ROWREG ? MRB : 1];
  auto rk_of = [&](int j) -> int {
    return ROWREG ? ri[ROWREG ? j : 0].rk : n_info[16 * (wr + RG * j) + m].rk;
  };
  // base logits of block j of the unit in slab sl, for this lane's 8 tokens
  auto fetch_base = [&](int j, int sl, u32x4_t& dst) {
    const int n = 16 * (wr + RG * j) + m;
    const int tgt = sl * SLAB + tw * TOK_PER_WAVE + 8 * g;
    dst = (u32x4_t){0u, 0u, 0u, 0u};
    if (j < my_nrb && n < rows && tgt < V)
      dst = *(const u32x4_t*)(a.base + (size_t)rk_of(j) * V + tgt);
  };

  const float mult = a.mult, cap = a.cap, inv_cap = a.inv_cap;
  const bool has_cap = a.has_cap != 0;
  // the transform table in LDS holds this launch's (mult, cap)
  const bool tt = tt_lay && (tts0 == TT_MAGIC) & (tts1 == __float_as_uint(mult)) &
                            (tts2 == __float_as_uint(cap));
  const float pinf = a.inf;
  float v1[MRB], v2[MRB];
  int idt[MRB];
  uint32_t spm = 0u;   // bit j: row block j has a non-finite estimate or logit
  // noisy rows of plans with registers to spare: the packed (high and low
  // half) largest |cached logit| bits, checked once at the end; the others
  // test every estimate
  constexpr bool PKMAX = MRB <= 4;
  uint32_t mxw[PKMAX ? MRB : 1];
  uint32_t lw[CARRY ? MRB : 1];   // noisy rows: the word of cached logits holding the top element's

  unsigned long long* slots_step = bias_mode ? nullptr : a.slots + (size_t)sset * SG * rows;
  unsigned long long* slots_cur = bias_mode ? nullptr : slots_step + (size_t)(blockIdx.x % SG) * rows;
  lds_barrier();
  if (ROWREG) {
#pragma unroll
    for (int j = 0; j < (ROWREG ? MRB : 1); ++j) ri[j] = n_info[j < my_nrb ? 16 * (wr + RG * j) + m : 0];
  }
  // base logits of the first unit
  if (!bias_mode && U > 0) {
#pragma unroll
    for (int j = 0; j < MRB; ++j) fetch_base(j, slab0, bq[j]);
  }

  // 4. the embeddings, straight into LDS (16-byte chunks, swizzled);
  //    padding rows read row 0 and are never used
  {
    const int total = rp * cpr;
    for (int j = wave; j * 64 < total; j += NWV) {
      const int p = j * 64 + lane;
      if (p < total) {
        const int n = p / cpr, cs = p - n * cpr;
        const uint16_t* src = a.w1 + (size_t)n_src[n] * R + ((cs ^ (n & swz)) * 8);
        __builtin_amdgcn_global_load_lds((const void*)src,
                                         (__attribute__((address_space(3))) void*)(emb + (size_t)j * 512),
                                         16, 0, 0);
      }
    }
  }
  // the second tile in flight (two-tile waves), and the first of a wave that
  // did not request it above, issued after the gather so that waiting for
  // the gather does not wait for them (the compiler, which cannot tell that
  // the two requests of the first tile exclude each other, waits for the
  // gather before the later one)
  __builtin_amdgcn_sched_barrier(0);
  // (one-tile waves that did not request their first tile above do so after
  // the prologue's barrier: kept out of the burst the barrier waits on, it
  // streams while the SIMD's first wave computes)
  if (!tile_first && NB == 2) tile(0, (U > 0 ? slab0 : 0) * SLAB + tw * TOK_PER_WAVE);
  __builtin_amdgcn_sched_barrier(0);
  if (NB == 2) tile(NB - 1, (U > 1 ? slab0 + slab_step : 0) * SLAB + tw * TOK_PER_WAVE);
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int j = 0; j < MRB; ++j) {
    v1[j] = -INFINITY;
    v2[j] = -INFINITY;
    idt[j] = NONE;
    if (PKMAX) mxw[PKMAX ? j : 0] = 0u;
    if (CARRY) lw[CARRY ? j : 0] = 0u;
  }
  // everything but the tiles requested after the gather: the embeddings
  // (every wave's, hence the barrier), the table, base logits and a first
  // tile requested before the gather (a count past the field's 63 waits for
  // more, never for less)
  constexpr int VM_FIRST = NB == 2 ? 2 * KB : 0;
  constexpr int VM_AFTER = NB == 2 ? (NB * 2 * KB < 63 ? NB * 2 * KB : 63) : 0;
  if (tile_first) wait_vm<VM_FIRST>();
  else wait_vm<VM_AFTER>();
  lds_barrier();
  if (!tile_first && NB == 1 && U > 0) tile(0, slab0 * SLAB + tw * TOK_PER_WAVE);
  if (tid < rp) acc_v2[tid] = order_key(-INFINITY);   // n_src is read by the gather only

  // one 32-token unit (the wave's unit i, slab `sl`) with w2 tile buffer BUF
  auto unit = [&](auto bufc, int i, int sl) {
    constexpr int BUF = decltype(bufc)::value;
    // an opaque zero added to the row blocks' embedding offsets: with many
    // row blocks the compiler would otherwise keep every block's operand
    // addresses across the unit loop, more than the registers hold
    int z0 = 0;
    if (MRB > 4) asm volatile("" : "+s"(z0));
    const int tok0 = sl * SLAB + tw * TOK_PER_WAVE;
    const int tg = tok0 + 8 * g;               // this lane's 8 tokens: tg .. tg+7
    const bool tok_ok = tg < V;
    const bool ntile = i + NB < U;             // the unit whose tile goes into this buffer next
    const int nsl = sl + NB * slab_step;
    const bool pnext = i + 1 < U;              // the next unit (base logit prefetch)
    const int psl = sl + slab_step;
    uint32_t kw[8];
    if (!bias_mode && !GREEDY) {
      uint32_t kc = (uint32_t)(tg + gofs) * MM_C1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kw[e] = rotl32(rotl32(kc, 15) * MM_C2, 13);   // the token word, rotated for mm_finish_rot
        kc += MM_C1;
      }
    }
    // E4M3 w2: this unit's codes to operands, its tokens' scales to binary32;
    // with two raw buffers the buffer's next tile goes out at once
    constexpr int AB = W8 ? 0 : BUF;           // the operand buffer of this unit
    f32x4_t sc0 = (f32x4_t){1.f, 1.f, 1.f, 1.f}, sc1 = sc0;
    if constexpr (W8) {
      decode_w2q_tile<KB>(Qa[BUF], Qb[BUF], A0[0], A1[0]);
      const u32x4_t S = QS[BUF];
      sc0 = (f32x4_t){f16_lo(S.x), f16_hi(S.x), f16_lo(S.y), f16_hi(S.y)};
      sc1 = (f32x4_t){f16_lo(S.z), f16_hi(S.z), f16_lo(S.w), f16_hi(S.w)};
      if (NB == 2 && ntile) tile(BUF, nsl * SLAB + tw * TOK_PER_WAVE);
    }
    constexpr bool LATE = !(W8 && NB == 2);    // the next tile after the unit's last contraction
    f32x4_t cb0[MRB], cb1[MRB];
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < my_nrb)
        block_bias<KB, W8>(A0[AB], A1[AB], emb, 16 * (wr + RG * j) + z0, m, R, g, swz, kzero, cb0[j], cb1[j]);
    if (LATE && D > 0 && my_nrb <= D && ntile) tile(BUF, nsl * SLAB + tw * TOK_PER_WAVE);
#pragma unroll
    for (int j = 0; j < MRB; ++j) {
      const int n = 16 * (wr + RG * j) + m;
      // block j's base logits of the next unit (a whole unit ahead). With
      // one row group of 2 or 4 bf16 blocks they are requested before the
      // contraction below: after it, the copy that hands the loop-carried
      // registers over waits for every load in flight, the next tile
      // included, which the contraction of the unit's last block has just
      // requested; before it, the tile streams through the unit's element
      // work. (Measured: the other plans, E4M3 ones included, are as fast
      // or faster with the request after the contraction, where the earlier
      // requests do not queue ahead of the tile, vector memory completing in
      // issue order.)
      constexpr bool EARLY_BASE = RG == 1 && (MRB == 2 || MRB == 4) && !W8;
      u32x4_t bv;
      if constexpr (EARLY_BASE) {
        bv = bq[j];
        if (!bias_mode && pnext) fetch_base(j, psl, bq[j]);
      }
      // the contraction of block j + D (of block j itself when D == 0);
      // once the unit's last one has issued, this buffer's next tile
      if (D == 0) {
        if (j < my_nrb) {
          block_bias<KB, W8>(A0[AB], A1[AB], emb, n - m + z0, m, R, g, swz, kzero, cb0[j], cb1[j]);
          if (LATE && j == my_nrb - 1 && ntile) tile(BUF, nsl * SLAB + tw * TOK_PER_WAVE);
        }
      } else if (j + D < MRB && j + D < my_nrb) {
        block_bias<KB, W8>(A0[AB], A1[AB], emb, n - m + 16 * RG * D + z0, m, R, g, swz, kzero, cb0[j + D], cb1[j + D]);
        if (LATE && j + D == my_nrb - 1 && ntile) tile(BUF, nsl * SLAB + tw * TOK_PER_WAVE);
      }
      if constexpr (!EARLY_BASE) {
        bv = bq[j];
        if (!bias_mode && pnext) fetch_base(j, psl, bq[j]);
      }
      if (j >= my_nrb) continue;

      const RowInfo info = ROWREG ? ri[ROWREG ? j : 0] : n_info[n];
      const bool active = n < rows && tok_ok;
      const bool noisy = !(info.T == 0.0f);
      f32x4_t c0 = cb0[j], c1 = cb1[j];
      if constexpr (W8) {                      // the row scale, one binary32 product
        c0 = c0 * sc0;
        c1 = c1 * sc1;
      }
      uint32_t bw[4];
      bw[0] = pack_bf16(c0[0], c0[1]);
      bw[1] = pack_bf16(c0[2], c0[3]);
      bw[2] = pack_bf16(c1[0], c1[1]);
      bw[3] = pack_bf16(c1[2], c1[3]);
      if (bias_mode) {
        if (active)
          *(uint4*)(a.bias_out + (size_t)n_row[n] * V + tg) = make_uint4(bw[0], bw[1], bw[2], bw[3]);
        continue;
      }
      // logits: bf16 add (one binary32 add, rounded), multiplier, soft cap
      const uint32_t bwd[4] = {bv.x, bv.y, bv.z, bv.w};
      uint32_t cw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        cw[q] = pack_bf16(bf_lo(bwd[q]) + bf_lo(bw[q]), bf_hi(bwd[q]) + bf_hi(bw[q]));
      if (has_cap && tt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) cw[q] = tt_map(cw[q]);
      } else if (has_cap) {
        float z[8];
        float zmax = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          z[2 * q] = (mult * bf_lo(cw[q])) * inv_cap;       // mult = 1: exact, no select
          z[2 * q + 1] = (mult * bf_hi(cw[q])) * inv_cap;
          zmax = fmaxf(zmax, fmaxf(fabsf(z[2 * q]), fabsf(z[2 * q + 1])));
        }
        if (__any(!(zmax < 0.625f))) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            cw[q] = pack_bf16(cap * tanh_fast(z[2 * q]), cap * tanh_fast(z[2 * q + 1]));
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            cw[q] = pack_bf16(cap * tanh_poly(z[2 * q]), cap * tanh_poly(z[2 * q + 1]));
        }
      } else if (mult != 1.0f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) cw[q] = pack_bf16(mult * bf_lo(cw[q]), mult * bf_hi(cw[q]));
      }
      float l[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        l[2 * q] = bf_lo(cw[q]);
        l[2 * q + 1] = bf_hi(cw[q]);
      }
      if (active && (!GREEDY || a.cache != nullptr))
        __builtin_nontemporal_store((u32x4_t){cw[0], cw[1], cw[2], cw[3]},
                                    (u32x4_t*)(a.cache + (size_t)info.rk * V + tg));
      if (GREEDY) {
        // the row's largest logit under the total order, exactly: elements
        // arrive in rising id, so an element wins over the kept one iff the
        // kept one is not NaN and the element is NaN or larger (a NaN is
        // kept from its first occurrence; ties keep the earlier id); the
        // first element of a row is taken whatever it is (so -inf too)
        if (active) {
          float x1 = v1[j];
          uint32_t e1 = __float_as_uint(v2[j]);
          bool have = idt[j] != NONE, upd = false;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool take = !have || (!__builtin_isnan(x1) && (__builtin_isnan(l[e]) || l[e] > x1));
            x1 = take ? l[e] : x1;
            e1 = take ? (uint32_t)e : e1;
            upd = upd || take;
            have = true;
          }
          if (upd) idt[j] = tg;
          v1[j] = x1;
          v2[j] = __uint_as_float(e1);
        }
        continue;
      }

      if (EXACT) {
        if (active) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float key = l[e];
            if (noisy) key = key_exact(l[e], info.T, mm_finish_rot(rotl32(info.prefix, 13), kw[e]));
            if (before(key, tg + e, v1[j], idt[j])) {
              v1[j] = key;
              idt[j] = tg + e;
            }
          }
        }
        continue;
      }
      // noisy rows: the two largest upper bounds, the element's index in
      // the tile packed into the bound's low 3 bits
      if (__any(active && noisy)) {
        if (active && noisy) {
          float x1 = v1[j], x2 = v2[j];
          const float x1b = x1;
          bool spx = false;
          // the largest magnitudes (bf16 bits, sign cleared), two per word
          if (PKMAX)
            mxw[PKMAX ? j : 0] = pk_max_u16(mxw[PKMAX ? j : 0],
                                            pk_max_u16(pk_max_u16(cw[0] & 0x7fff7fffu, cw[1] & 0x7fff7fffu),
                                                       pk_max_u16(cw[2] & 0x7fff7fffu, cw[3] & 0x7fff7fffu)));
          // all 8 table reads in flight before the first is used
          float fh[8];
          const uint32_t pr = rotl32(info.prefix, 13);
#pragma unroll
          for (int e = 0; e < 8; ++e) fh[e] = (float)mm_finish_rot(pr, kw[e]);
          float2 ab[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (LIN) ab[e] = gtab[gt_index(fh[e])];
            else ab[e].x = gtabf[gt_index(fh[e])];
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float gh = LIN ? __builtin_fmaf(ab[e].y, fh[e], ab[e].x) : ab[e].x;
            // the estimate fma(l, RN(1/T), bound); its margin for the
            // roundings and the packed index is added once per row (see
            // slack_up), as it grows with the estimate
            const float hi = __builtin_fmaf(l[e], info.rcp, gh);
            if (!PKMAX) spx = spx || __builtin_amdgcn_class(hi, 0x207);   // NaN or infinite
            const float pk = __uint_as_float((__float_as_uint(hi) & ~7u) | (uint32_t)e);
            x2 = __builtin_amdgcn_fmed3f(x1, x2, pk);
            x1 = __builtin_amdgcn_fmed3f(x1, pk, pinf);   // max, no canonicalising
          }
          if (x1 != x1b) {
            idt[j] = tg;
            if (CARRY) {
              const uint32_t e1 = __float_as_uint(x1);
              lw[CARRY ? j : 0] = (e1 & 4u) ? ((e1 & 2u) ? cw[3] : cw[2]) : ((e1 & 2u) ? cw[1] : cw[0]);
            }
          }
          v1[j] = x1;
          v2[j] = x2;
          if (!PKMAX) spm |= (spx ? 1u : 0u) << j;
        }
      }
      // temperature-0 rows: the exact largest logit, the earliest on ties
      // (elements arrive in rising id); v2 holds its index in the tile
      if (__any(active && !noisy)) {
        if (active && !noisy) {
          float x1 = v1[j];
          const float x1b = x1;
          uint32_t e1 = __float_as_uint(v2[j]);
          bool spx = false;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            spx = spx || __builtin_amdgcn_class(l[e], 0x007);   // NaN or -inf
            const bool gt = l[e] > x1;
            x1 = gt ? l[e] : x1;
            e1 = gt ? (uint32_t)e : e1;
          }
          if (x1 != x1b) idt[j] = tg;
          v1[j] = x1;
          v2[j] = __uint_as_float(e1);
          spm |= (spx ? 1u : 0u) << j;
        }
      }
    }
  };

  // the wave's units (a two-tile wave alternates its buffers)
  for (int i = 0; i < U; i += NB) {
    unit(std::integral_constant<int, 0>{}, i, slab0 + i * slab_step);
    if (NB == 2 && i + 1 < U) unit(std::integral_constant<int, NB - 1>{}, i + 1, slab0 + (i + 1) * slab_step);
  }
  if (bias_mode) return;

  // 5. each row's state. Every lane keeps one state per row block (its share
  //    of the row over the wave's units). It goes into the row's LDS
  //    accumulators: the winner's packed order key by a 64-bit atomic max
  //    (a lane's own re-scan flag by an atomic or) as soon as the wave leaves
  //    the slab loop; after one barrier, the second bound by a 32-bit atomic
  //    max of every other state's v1 and the winner's v2, and the winner's
  //    carried logit from its lane; after a second barrier, one thread per
  //    row takes the exact key of the winner and publishes it with the packed
  //    atomicMax, or lists the row for a re-scan.
  auto state_id = [&](int j, bool noisy) -> int {
    if (EXACT) return idt[j];
    if (idt[j] == NONE) return NONE;
    return idt[j] + (int)((noisy ? __float_as_uint(v1[j]) : __float_as_uint(v2[j])) & 7u);
  };
#pragma unroll
  for (int j = 0; j < MRB; ++j) {
    if (j >= my_nrb) continue;   // (not break: the loop stays a counted one, unrolled)
    const int n = 16 * (wr + RG * j) + m;
    const RowInfo info = ROWREG ? ri[ROWREG ? j : 0] : n_info[n];
    const bool noisy = !(info.T == 0.0f);
    // a noisy row's estimates fma(l, RN(1/T), bound) are all finite when
    // RN(|l| |RN(1/T)|) <= 2^127 for its largest |l| (the bound is finite
    // and under 2^5); else (a NaN or infinite logit, a NaN or infinite
    // 1/T, or a product past 2^127, where NaN compares false) re-scan it
    bool spn = false;
    if (PKMAX) {
      const uint32_t mh = mxw[PKMAX ? j : 0] >> 16, ml = mxw[PKMAX ? j : 0] & 0xffffu;
      const float lmax = __uint_as_float((mh > ml ? mh : ml) << 16);
      spn = noisy && !EXACT && !(lmax * fabsf(info.rcp) <= 0x1p127f);
    }
    const int id = state_id(j, noisy);
    if (id != NONE)
      __hip_atomic_fetch_max(acc_win + n, pack_winner(v1[j], id), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (((spm >> j) & 1u) | (spn ? 1u : 0u))
      __hip_atomic_fetch_or(acc_lsp + n, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  lds_barrier();
  if (!EXACT && !GREEDY) {
#pragma unroll
    for (int j = 0; j < MRB; ++j) {
      if (j >= my_nrb) continue;
      const int n = 16 * (wr + RG * j) + m;
      const RowInfo info = ROWREG ? ri[ROWREG ? j : 0] : n_info[n];
      if (info.T == 0.0f) continue;   // an ORDER row keeps no second bound
      const int id = state_id(j, true);
      const bool is_w = id != NONE && (uint32_t)acc_win[n] == ~(uint32_t)id;
      // a lane's v2 never exceeds its v1: the winner's lane gives its v2,
      // every other lane its v1
      const float c = is_w ? v2[j] : v1[j];
      if (c > -INFINITY)
        __hip_atomic_fetch_max(acc_v2 + n, order_key(c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (CARRY && is_w)
        __hip_atomic_fetch_or(acc_lsp + n,
                              (__float_as_uint(v1[j]) & 1u) ? (lw[CARRY ? j : 0] & 0xffff0000u) : (lw[CARRY ? j : 0] << 16),
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  if (tid == 0) misc[16] = 0;
  // without carried logits the winner's is read back from the cache below:
  // every wave's cache stores first
  const bool reads_cache = !(CARRY || GREEDY);
  if (reads_cache) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  } else {
    lds_barrier();
  }
  static_assert(ROWS_CAP <= NTH, "one thread per row");
  if (tid < rows) {
    const int n = tid;
    const RowInfo info = n_info[n];
    const bool noisy = !(info.T == 0.0f);
    const bool top2 = noisy && !EXACT;
    const unsigned long long w = acc_win[n];
    const int st_id = w == 0ull ? NONE : (int)~(uint32_t)w;
    const float st_v1 = order_value((uint32_t)(w >> 32));
    const int rr = n_row[n];
    float key = st_v1;
    bool fb = !EXACT && ((acc_lsp[n] & 1u) != 0u || (mode == MODE_SAMPLE_FALLBACK && noisy));
    float thr = -INFINITY;
    if (!fb && top2 && st_id != NONE) {
      float l1 = __uint_as_float(acc_lsp[n] & 0xffff0000u);
      if (!CARRY) {
        const size_t e = (size_t)info.rk * V + st_id;
        const uint32_t wd = load_cache_word(a.cache, e & ~(size_t)1);
        l1 = (e & 1) ? bf_hi(wd) : bf_lo(wd);
      }
      key = key_exact(l1, info.T, mm_finish(info.prefix, mm_token_word((uint32_t)(st_id + gofs))));
      const float v2u = slack_up(order_value(acc_v2[n]));
      if (!(key > v2u)) {
        // not certified: some other element's bound reaches the key. If a
        // key already published for this row (by another workgroup) lies
        // above that bound, no element here but the top one can win, and
        // the top one is published below; else re-scan the row.
        unsigned long long cur = 0ull;
        for (int q = 0; q < SG; ++q) {
          const unsigned long long c =
              __hip_atomic_load(slots_step + (size_t)q * rows + rr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          cur = c > cur ? c : cur;
        }
        if (!((uint32_t)(cur >> 32) > (uint32_t)(pack_winner(v2u, 0) >> 32))) {
          fb = true;
          thr = key;
        }
      }
    }
    if (fb) {
      const int i = atomicAdd(&misc[16], 1);
      fb_row[i] = n;
      fb_thr[i] = thr;
    } else if (st_id != NONE) {
      __hip_atomic_fetch_max(slots_cur + rr, pack_winner(key, st_id + gofs), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  lds_barrier();

  // 6. fallback rows, one per wave at a time: the wave re-reads the row's
  //    cached logits over the workgroup's slabs and takes the exact key of
  //    every element whose bound reaches the threshold (all of them for a
  //    row with a non-finite estimate). Only then does the workgroup wait
  //    for its cache stores (they are read back); otherwise they drain as
  //    the kernel ends.
  const int nfb = misc[16];
  if (nfb > 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  const int wg_slabs = (int)blockIdx.x < nslabs ? (nslabs - (int)blockIdx.x + G - 1) / G : 0;
  for (int f = wave; f < nfb; f += NWV) {
    const int n = fb_row[f];
    const float thr = fb_thr[f];
    const RowInfo info = n_info[n];
    const bool noisy = !(info.T == 0.0f);
    const int rr = n_row[n];
    float bv = -INFINITY;
    int bi = NONE;
    // once some element of the row has a NaN key (a NaN logit or
    // temperature, or an infinite logit over an infinite temperature; the
    // noise term is always finite), only the lowest such id can win, and no
    // other key is needed
    bool nan_mode = false;
    // the lane's words, FB_BATCH loads in flight at a time
    const int nq = wg_slabs * (SLAB / 2);
    for (int q0 = 0; q0 < nq; q0 += 64 * FB_BATCH) {
      uint32_t wd[FB_BATCH];
      int t0[FB_BATCH];
#pragma unroll
      for (int b = 0; b < FB_BATCH; ++b) {
        const int q = q0 + 64 * b + lane;
        t0[b] = q < nq ? ((int)blockIdx.x + (q / (SLAB / 2)) * G) * SLAB + 2 * (q % (SLAB / 2)) : V;
        wd[b] = t0[b] < V ? load_cache_word(a.cache, (size_t)info.rk * V + t0[b]) : 0u;
      }
      // with a threshold: the elements whose bound reaches it, the first two
      // of the lane's kept aside and their exact keys taken together below
      int nc = 0, ct0 = 0, ct1 = 0;
      float cl0 = 0.0f, cl1 = 0.0f;
      uint32_t ch0 = 0u, ch1 = 0u;
      const bool screen = noisy && !(thr == -INFINITY);
      if (noisy && !screen) {
        bool any_nan = false;
#pragma unroll
        for (int b = 0; b < FB_BATCH; ++b) {
          if (t0[b] >= V) continue;
          any_nan = any_nan || key_is_nan(bf_lo(wd[b]), info.T) || key_is_nan(bf_hi(wd[b]), info.T);
        }
        nan_mode = nan_mode || __any(any_nan);
      }
#pragma unroll
      for (int b = 0; b < FB_BATCH; ++b) {
        if (t0[b] >= V) continue;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int t = t0[b] + e;
          const float l = e ? bf_hi(wd[b]) : bf_lo(wd[b]);
          if (screen) {
            const uint32_t h = mm_finish(info.prefix, mm_token_word((uint32_t)(t + gofs)));
            if (!(key_upper(l, info.rcp, noise_bound<LIN>(gtab, h)) < thr)) {
              if (nc == 0) {
                ct0 = t;
                cl0 = l;
                ch0 = h;
              } else if (nc == 1) {
                ct1 = t;
                cl1 = l;
                ch1 = h;
              }
              ++nc;
            }
          } else {
            float key = l;
            if (noisy && nan_mode)
              key = key_is_nan(l, info.T) ? __builtin_nanf("") : -INFINITY;
            else if (noisy)
              key = key_exact(l, info.T, mm_finish(info.prefix, mm_token_word((uint32_t)(t + gofs))));
            if (before(key, t, bv, bi)) {
              bv = key;
              bi = t;
            }
          }
        }
      }
      if (nc > 0) {
        const float key = key_exact(cl0, info.T, ch0);
        if (before(key, ct0, bv, bi)) {
          bv = key;
          bi = ct0;
        }
      }
      if (nc > 1) {
        const float key = key_exact(cl1, info.T, ch1);
        if (before(key, ct1, bv, bi)) {
          bv = key;
          bi = ct1;
        }
      }
      if (nc > 2) {   // rare: every candidate of the batch, again
#pragma unroll
        for (int b = 0; b < FB_BATCH; ++b) {
          if (t0[b] >= V) continue;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int t = t0[b] + e;
            const float l = e ? bf_hi(wd[b]) : bf_lo(wd[b]);
            const uint32_t h = mm_finish(info.prefix, mm_token_word((uint32_t)(t + gofs)));
            if (key_upper(l, info.rcp, noise_bound<LIN>(gtab, h)) < thr) continue;
            const float key = key_exact(l, info.T, h);
            if (before(key, t, bv, bi)) {
              bv = key;
              bi = t;
            }
          }
        }
      }
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const float ov = __shfl_xor(bv, sh);
      const int oi = __shfl_xor(bi, sh);
      if (before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0 && bi != NONE)
      __hip_atomic_fetch_max(slots_cur + rr, pack_winner(bv, bi + gofs), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }

  // 7. the last step (and every step of a vocabulary shard): the workgroup
  //    that finishes last turns the winners into tokens[:, k-1] (a shard's
  //    into its packets, the packed winner with the global id) and leaves
  //    every slot and the ticket zeroed for the next call. Every wave waits
  //    for its own slot atomics (vmcnt(0)) before the workgroup barrier;
  //    thread 0 then takes the ticket with an agent-scope release fetch-add,
  //    so the workgroup's slot updates are visible at agent scope before its
  //    ticket counts, and the workgroup that takes the last ticket executes
  //    an agent-scope acquire fence before it reads the slots (the
  //    acquire-release pairing of the HIP / AMDGPU memory model). Nothing
  //    waits on another workgroup.
  if (shard || s == K - 1) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      misc[17] = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) ==
                         (unsigned)G - 1u
                     ? 1
                     : 0;
    __syncthreads();
    if (misc[17]) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      unsigned long long* fin_slots = a.slots + (size_t)sset * SG * rows;
      for (int r2 = tid; r2 < rows; r2 += NTH) {
        unsigned long long w = 0ull;
#pragma unroll
        for (int q = 0; q < SG; ++q) {
          const unsigned long long c = __hip_atomic_exchange(fin_slots + (size_t)q * rows + r2, 0ull,
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          w = c > w ? c : w;
        }
        if (shard) {
          a.packets[r2] = w;
        } else {
          a.tokens[(int64_t)r2 * K + K - 1] = slot_token(w);
          if (a.winners) a.winners[(int64_t)r2 * K + K - 1] = w;
        }
      }
      for (int i = tid; i < 3 * SG * rows; i += NTH)
        if (i / (SG * rows) != sset) a.slots[i] = 0ull;
      if (tid == 0) __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// One kernel of the step for a rank class KB and a plan (row groups, row
// blocks per wave); nullptr for a plan the rank class does not build.
template <int KB, int VAR>
StepFn pick_plan(int rg, int mrb) {
  if (rg == 1) {
    switch (mrb) {
      case 1: return markov_step_kernel<KB, 1, 1, VAR>;
      case 2: return markov_step_kernel<KB, 1, 2, VAR>;
      case 4: return markov_step_kernel<KB, 1, 4, VAR>;
      case 8: return markov_step_kernel<KB, 1, 8, VAR>;
    }
  } else if (rg == 2) {
    switch (mrb) {
      case 8: return markov_step_kernel<KB, 2, 8, VAR>;
      case 16:
        if constexpr (KB <= 8) return markov_step_kernel<KB, 2, 16, VAR>;
        break;
    }
  }
  return nullptr;
}

}  // namespace

// The step kernels of each (rank class, variant) are compiled in a translation
// unit of their own (step_inst.hip built once per pair); each returns its
// kernel for a plan. X(KB, VAR) lists the pairs built.
#define MARKOV_STEP_INSTANCES(X) \
  X(1, 0) X(1, 1) X(1, 2) X(1, 4) X(1, 6) X(2, 0) X(2, 1) X(2, 2) X(2, 4) X(2, 6) \
  X(4, 0) X(4, 1) X(4, 2) X(4, 4) X(4, 6) X(8, 0) X(8, 1) X(8, 2) X(8, 4) X(8, 6) \
  X(16, 0) X(16, 1) X(16, 2) X(16, 4) X(16, 6)

namespace markov_impl {
#define MARKOV_DECLARE_PICKER(KB, VAR) StepFn step_kernel_kb##KB##_v##VAR(int rg, int mrb);
MARKOV_STEP_INSTANCES(MARKOV_DECLARE_PICKER)
#undef MARKOV_DECLARE_PICKER
}  // namespace markov_impl
