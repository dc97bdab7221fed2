// MI355X (gfx950, CDNA4) DSpark sequential Markov draft-sampling step.
//
// One kernel launch per draft step. Every workgroup owns vocabulary slabs of
// SLAB tokens (persistently, grid-strided) and all request rows:
//   * the rows' Markov embeddings w1[prev] sit in LDS (16-byte chunks,
//     XOR-swizzled by row so the MFMA operand reads hit distinct banks);
//   * each wave streams its 32 tokens' w2 rows from HBM once per step,
//     straight into v_mfma_f32_16x16x32_bf16 A operands (16-byte loads);
//     tokens sit on the MFMA's M side, in an order chosen so that after the
//     MFMA each lane holds 8 consecutive tokens of one row, so the base read
//     and the cache write are 16-byte vectors with no LDS transpose;
//   * the epilogue (bf16 bias, bf16 add, multiplier / soft cap, cache store)
//     and the Gumbel noise run in registers; a cheap noise estimate with a
//     proven error margin decides which elements can still win, and only
//     those get the exact key (binary64 logs, IEEE division);
//   * per-row winners go out as one packed (order-preserving key, ~id)
//     64-bit atomicMax per row per workgroup; the last workgroup to arrive
//     writes tokens[:, step] and re-zeroes the slots and the counter.
//
// The definition followed is stated in include/markov.h, with the pages it
// comes from (vLLM Markov-drafter API pages: kimi_k3 `_gumbel_key` and the
// module's exactness paragraph; muse_spark cutedsl `_logit`, `_gumbel`,
// `_murmur_prefix`, `_combine`, `_w1_row`, `_StepKernel.kernel`).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "markov.h"

namespace {

constexpr int NW = 4;                  // waves per workgroup
constexpr int BLOCK = 64 * NW;         // threads per workgroup
constexpr int TOK_PER_WAVE = 32;       // two 16-token MFMA M tiles
constexpr int SLAB = NW * TOK_PER_WAVE;
constexpr int NONE = 0x7fffffff;       // id of "no element yet"
constexpr int LDS_EMB_MAX = 128 * 1024;
constexpr int ROWS_CAP = 1024;

enum Mode { MODE_SAMPLE = 0, MODE_SAMPLE_EXACT = 1, MODE_BIAS = 2, MODE_SAMPLE_FALLBACK = 3 };

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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
  unsigned long long* slots;  // [3][rows] packed winners, step s uses s % 3
  uint16_t* bias_out;
  int rows, V, R, k, step, nslabs, mode;
  float mult, inv_cap, cap;
  int has_cap;
};

// ---------------------------------------------------------------- numbers

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two binary32 -> one word of two bf16 (round to nearest even; the hardware
// conversion v_cvt_pk_bf16_f32), `a` in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
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

__device__ __forceinline__ uint32_t mm_finish(uint32_t prefix, uint32_t token_word) {
  uint32_t h = prefix ^ token_word;
  h = rotl32(h, 13);
  h = (h << 2) + h + 0xe6546b64u;   // h * 5 + c
  h ^= 16u;                       // message length in bytes
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
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
__device__ __forceinline__ float uniform_of(uint32_t h) {
  float hi = (float)(h >> 16), lo = (float)(h & 0xffffu);
  return __builtin_fmaf(hi, 0x1p-16f, __builtin_fmaf(lo, 0x1p-32f, 0x1p-33f));
}

// ---------------------------------------------------------------- keys
// Exact key: RN32(RN32(l / T) - lb), lb = RN32(log(-L)), L = log(1 - u) in
// the pages' stable form (a Horner series below u = 1/4, else a log of
// max(1 - u, 2^-24)). Logs are taken in binary64 and rounded once.
__device__ __forceinline__ float log1m_exact(float u) {
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

__device__ __noinline__ float key_exact(float l, float T, uint32_t h) {
  float u = uniform_of(h);
  float L = log1m_exact(u);
  float lb = (float)log((double)(-L));
  float q = l / T;
  return q - lb;
}

// Cheap key estimate. The uniform is taken with one conversion (within
// 2^-23 relative of the exact one); y2 = -log2(1 - u) by u (1 + u/2) / ln 2
// below u = 2^-10, else by the hardware log2 of max(1 - u, 2^-24); then
// key ~ l / T - ln(y2 ln 2) = l rcp(T) + (-ln ln 2) - ln2 log2(y2).
// |key_fast - key_exact| <= 1e-3 + |key_fast| 2^-18 (the margin the kernel
// trusts; the tests check it against the exact key over many hashes): the
// estimate's own error is below 1e-4 plus a few ulps of |l / T| <= |key| + 23.
constexpr float LN2F = 0.693147180559945309f;
constexpr float LOG2EF = 1.44269504088896341f;
constexpr float NEG_LN_LN2 = 0.366512920581664327f;

__device__ __forceinline__ float key_fast(float l, float rcpT, uint32_t h) {
  const float u = __builtin_fmaf((float)h, 0x1p-32f, 0x1p-33f);
  const float ys = u * __builtin_fmaf(u, 0.5f * LOG2EF, LOG2EF);
  const float yl = -__builtin_amdgcn_logf(fmaxf(1.0f - u, 0x1p-24f));
  const float y2 = u < 0x1p-10f ? ys : yl;
  const float qc = __builtin_fmaf(l, rcpT, NEG_LN_LN2);
  return __builtin_fmaf(-LN2F, __builtin_amdgcn_logf(y2), qc);
}

__device__ __forceinline__ float fast_margin(float ka) { return __builtin_fmaf(fabsf(ka), 0x1p-18f, 1e-3f); }

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

template <typename T8>
__device__ __forceinline__ T8 pick8(const T8* v, int e) {
  T8 r = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) r = (e == i) ? v[i] : r;
  return r;
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *(const uint4*)p; }

// ---------------------------------------------------------------- the step

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// The winner slot of a row decodes to its token id.
__device__ __forceinline__ int64_t slot_token(unsigned long long w) {
  return (int64_t)(uint32_t)(~(uint32_t)w);
}

// Merge rules of the per-row states. ORDER: the exact (key, id) under the
// total order. TOP2: (v1, id1, l1) is the element with the largest upper
// bound v1 of its key, v2 the largest upper bound among all other elements.
struct RowState {
  float v1, v2, l1;
  int id1;
};

__device__ __forceinline__ void merge_order(RowState& a, const RowState& b) {
  if (before(b.v1, b.id1, a.v1, a.id1)) {
    a.v1 = b.v1;
    a.id1 = b.id1;
    a.l1 = b.l1;
  }
}

__device__ __forceinline__ void merge_top2(RowState& a, const RowState& b) {
  const bool bw = (b.v1 > a.v1) || (b.v1 == a.v1 && b.id1 < a.id1);
  const float lose = bw ? a.v1 : b.v1;
  const float win2 = bw ? b.v2 : a.v2;
  a.v2 = fmaxf(lose, win2);
  if (bw) {
    a.v1 = b.v1;
    a.id1 = b.id1;
    a.l1 = b.l1;
  }
}

// Upper bound of an exact key from its estimate, less the constant part of
// the margin (added back at the decision): key <= hi + 1e-3.
__device__ __forceinline__ float upper_of(float ka) { return __builtin_fmaf(fabsf(ka), 0x1p-18f, ka); }

// Lower bound of the exact key of the element whose upper bound is v1:
// key >= v1 - 2 * margin, with margin = 1e-3 + |ka| 2^-18 (rounded up).
__device__ __forceinline__ float lower_of_upper(float v1) {
  return v1 - 2.5e-3f - fabsf(v1) * 0x1p-16f;
}

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
      A0[i] = __builtin_nontemporal_load((const bf16x8_t*)(pa + ch * 8));
      A1[i] = __builtin_nontemporal_load((const bf16x8_t*)(pb + ch * 8));
    }
  }
}

// tanh for the soft cap: an odd minimax polynomial z + z^3 P(z^2) below
// |z| = 0.625 (fitted here for binary32 Horner evaluation, within 0.7 ulp),
// else 1 - 2 / (e^{2|z|} + 1) with the hardware exp2 and reciprocal (about
// 2 ulp). The cache rounds the result to bf16.
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

// Per-lane view of one of the wave's row blocks, kept in registers for the
// whole step: the row's offset into base/cache, 1/T, the hash prefix, its
// kind, and the running state of this lane's elements of the row.

// Per LDS row n, one 16-byte record: rk = row * k + step (the row's slice of
// base / cache starts at rk * V), 1/T, the hash prefix and T.
struct RowInfo {
  int rk;
  float rcp;
  uint32_t prefix;
  float T;
};
typedef RowInfo RowInfoReg;
struct LaneRow {
  float v1, v2, l1;
  int id1;
  RowInfoReg info;   // the row's constants, when kept in registers
};
constexpr int PFD = 2;  // base logits are requested this many row blocks ahead

// The bias of one 16-row block for the wave's 32 tokens: lane (g, m) gets
// row n = 16 rb + m, tokens tg .. tg+3 in c0 and tg+4 .. tg+7 in c1.
template <int KB>
__device__ __forceinline__ void block_bias(const bf16x8_t* A0, const bf16x8_t* A1, const uint16_t* emb,
                                           int n, int R, int g, int swz, bool kzero, f32x4_t& c0,
                                           f32x4_t& c1) {
  c0 = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  c1 = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KB; ++i) {
    bf16x8_t B;
    if (kzero) {
      B = (bf16x8_t){};
    } else {
      const int ch = 4 * i + g;
      B = *(const bf16x8_t*)(emb + (size_t)n * R + ((ch ^ (n & swz)) * 8));
    }
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[i], B, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[i], B, c1, 0, 0, 0);
  }
}

// Waves: 4 token waves (32 tokens each, a 128-token slab) times RG row
// groups; the wave's row blocks are rb = wr + j RG, j < MRB (unrolled, so
// their state lives in registers). Row groups share the workgroup's LDS copy
// of the embeddings.
template <int KB, int RG, int MRB, bool EXACT>
__global__ __launch_bounds__(256 * RG) void markov_step_kernel(StepArgs a) {
  constexpr int NWV = 4 * RG;                   // waves per workgroup
  constexpr int NTH = 64 * NWV;
  extern __shared__ __align__(16) unsigned char lds[];
  const int mode = a.mode;
  const bool bias_mode = mode == MODE_BIAS;
  constexpr bool exact_mode = EXACT;   // the test-only exact-everywhere variant
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wt = wave & 3, wr = wave >> 2;
  const int g = lane >> 4, m = lane & 15;
  const int R = KB >= 2 ? 32 * KB : a.R;         // the rank is fixed by KB from 64 up
  const int rows = a.rows, rp = (rows + 15) & ~15, V = a.V, s = a.step, K = a.k;
  const int cpr = R >> 3;                       // 16-byte chunks per embedding row
  const int swz = (cpr < 16 ? cpr : 16) - 1;   // a 16-lane LDS pass reads 16 distinct chunks
  const int G = gridDim.x;

  uint16_t* emb = (uint16_t*)lds;
  RowInfo* n_info = (RowInfo*)(lds + (size_t)rp * R * 2);  // by LDS row n
  int* n_row = (int*)(n_info + rp);                // LDS row n -> request row
  int* n_src = n_row + rp;                         // its w1 row
  float* st_v1 = (float*)(n_src + rp);             // [4][rp] row states, by token wave
  float* st_v2 = st_v1 + 4 * rp;
  float* st_l = st_v2 + 4 * rp;
  int* st_id = (int*)(st_l + 4 * rp);
  int* sp_cnt = st_id + 4 * rp;                    // [rp] elements whose estimate is not finite
  int* fb_list = sp_cnt + rp;                      // [rp] rows that take the exact fallback
  int* misc = fb_list + rp;                        // chunk counts [2][16], fallback count

  unsigned long long* slots_cur = a.slots ? a.slots + (size_t)(s % 3) * rows : nullptr;
  const unsigned long long* slots_prev = a.slots ? a.slots + (size_t)((s + 2) % 3) * rows : nullptr;
  unsigned long long* slots_next = a.slots ? a.slots + (size_t)((s + 1) % 3) * rows : nullptr;

  // 1. rows: the token feeding this step (decoded from the previous step's
  //    winner slots), temperature, hash prefix. Noisy rows are placed first
  //    so that 16-row blocks are of one kind.
  const int nchunks = (rows + 63) >> 6;
  for (int c = wave; c < nchunks; c += NWV) {
    const int r = c * 64 + lane;
    const bool valid = r < rows;
    const float T = (!bias_mode && valid) ? a.temperature[r] : 0.0f;
    const bool noisy = valid && !(T == 0.0f);
    const uint64_t bn = __ballot(noisy), bz = __ballot(valid && !noisy);
    if (lane == 0) {
      misc[c] = __builtin_popcountll(bn);
      misc[16 + c] = __builtin_popcountll(bz);
    }
  }
  for (int n = rows + tid; n < rp; n += NTH) {
    n_row[n] = 0;
    n_src[n] = 0;
    n_info[n] = RowInfo{s, 0.0f, 0u, 0.0f};
  }
  for (int n = tid; n < rp; n += NTH) sp_cnt[n] = 0;
  if (tid == 0) misc[32] = 0;
  __syncthreads();
  int total_noisy = 0;
  for (int c = 0; c < nchunks; ++c) total_noisy += misc[c];
  for (int c = wave; c < nchunks; c += NWV) {
    const int r = c * 64 + lane;
    const bool valid = r < rows;
    float T = 0.0f;
    int64_t t = 0;
    if (valid) {
      if (!bias_mode) T = a.temperature[r];
      t = (bias_mode || s == 0) ? a.prev[r] : slot_token(slots_prev[r]);
    }
    const bool noisy = valid && !(T == 0.0f);
    const uint64_t bn = __ballot(noisy), bz = __ballot(valid && !noisy);
    int pre_n = 0, pre_z = 0;
    for (int c2 = 0; c2 < c; ++c2) {
      pre_n += misc[c2];
      pre_z += misc[16 + c2];
    }
    if (valid) {
      const int pos = bias_mode ? r
                    : noisy ? pre_n + (int)lanes_below(bn)
                            : total_noisy + pre_z + (int)lanes_below(bz);
      const uint64_t ut = (uint64_t)t, last = (uint64_t)(V - 1);
      n_row[pos] = r;
      n_src[pos] = (int)(ut < last ? ut : last);
      n_info[pos] = RowInfo{r * K + s, 1.0f / T,
                            bias_mode ? 0u : row_prefix_of(a.seeds[r], s, a.positions[(int64_t)r * K + s]),
                            T};
      if (!bias_mode && blockIdx.x == 0) {
        if (s > 0) a.tokens[(int64_t)r * K + s - 1] = t;   // the previous step's token
        slots_next[r] = 0ull;                             // next step's slots start empty
      }
    }
  }
  __syncthreads();

  // 2. gather the embeddings straight into LDS (16-byte chunks, swizzled);
  //    padding rows read row 0 and are never used.
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

  // this lane's rows, one per row block of the wave
  const int nrb = rp >> 4;
  const int my_nrb = nrb > wr ? (nrb - wr + RG - 1) / RG : 0;
  // small row-block counts keep each row's constants in registers (they feed
  // the base-logit addresses); large ones read them from LDS per tile
  constexpr bool ROWREG = MRB <= 4;
  LaneRow lr[MRB];
#pragma unroll
  for (int j = 0; j < MRB; ++j) {
    if (ROWREG) {
      const int n = (wr + j * RG) * 16 + m;
      lr[j].info = n_info[j < my_nrb ? n : 0];
    }
    lr[j].v1 = -INFINITY;
    lr[j].v2 = -INFINITY;
    lr[j].l1 = 0.0f;
    lr[j].id1 = NONE;
  }
  const bool kzero = (KB == 1) && (R == 16) && (g >= 2);
  bf16x8_t A0[KB], A1[KB];
  int slab = blockIdx.x;
  if (my_nrb > 0) load_w2_tile<KB>(a.w2, V, R, slab * SLAB + wt * TOK_PER_WAVE, m, g, kzero, A0, A1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // D: row blocks whose contraction is issued ahead of the current epilogue;
  // once the slab's last contraction is out, the next slab's w2 tile is
  // requested, so it streams in under the remaining epilogues.
#ifndef MARKOV_AHEAD
#define MARKOV_AHEAD 1
#endif
#ifndef MARKOV_XSLAB
#define MARKOV_XSLAB 0
#endif
  constexpr int D = MRB - 1 < MARKOV_AHEAD ? MRB - 1 : MARKOV_AHEAD;
  const float mult = a.mult, cap = a.cap, inv_cap = a.inv_cap;
  u32x4_t bq[MRB];
  if (my_nrb > 0) {
    for (; slab < a.nslabs; slab += G) {
      if (!MARKOV_XSLAB || slab == (int)blockIdx.x) {
        const int tg0 = slab * SLAB + wt * TOK_PER_WAVE + 8 * g;
#pragma unroll
        for (int j = 0; j < MRB; ++j) {
          bq[j] = (u32x4_t){0u, 0u, 0u, 0u};
          const int n = (wr + j * RG) * 16 + m;
          if (!bias_mode && j < PFD && j < my_nrb && n < rows && tg0 < V)
            bq[j] = __builtin_nontemporal_load(
                (const u32x4_t*)(a.base + (size_t)(ROWREG ? lr[j].info.rk : n_info[n].rk) * V + tg0));
        }
      }
      const int tok0 = slab * SLAB + wt * TOK_PER_WAVE;
      const int nxt = slab + G;
      const int tg = tok0 + 8 * g;              // this lane's 8 tokens: tg .. tg+7
      const int tgn = tg + G * SLAB;            // the same lane's tokens in the next slab
      const bool tok_ok = tg < V, tokn_ok = nxt < a.nslabs && tgn < V;
      if (tok0 >= V) continue;                  // wave-uniform: the last slab's tail
      uint32_t kw[8];
      if (!bias_mode) {
#pragma unroll
        for (int e = 0; e < 8; ++e) kw[e] = mm_token_word((uint32_t)(tg + e));
      }
      f32x4_t cb0[MRB], cb1[MRB];
      bool a_out = false;                       // next slab's tile requested
#pragma unroll
      for (int j = 0; j < D; ++j)
        if (j < my_nrb) block_bias<KB>(A0, A1, emb, (wr + j * RG) * 16 + m, R, g, swz, kzero, cb0[j], cb1[j]);
      if (my_nrb <= D && nxt < a.nslabs) {
        load_w2_tile<KB>(a.w2, V, R, nxt * SLAB + wt * TOK_PER_WAVE, m, g, kzero, A0, A1);
        a_out = true;
      }
#pragma unroll
      for (int j = 0; j < MRB; ++j) {
        if (j >= my_nrb) break;
        const int n = (wr + j * RG) * 16 + m;
        if (j + D < MRB && j + D < my_nrb) {
          block_bias<KB>(A0, A1, emb, n + D * RG * 16, R, g, swz, kzero, cb0[j + D], cb1[j + D]);
          if (j + D == my_nrb - 1 && nxt < a.nslabs) {
            load_w2_tile<KB>(a.w2, V, R, nxt * SLAB + wt * TOK_PER_WAVE, m, g, kzero, A0, A1);
            a_out = true;
          }
        }
        // base logits PFD row blocks ahead, into the next slab past the end
        if (!bias_mode) {
          if (j + PFD < MRB) {
            const int n2 = n + PFD * RG * 16;
            if (n2 < rows && tok_ok && j + PFD < my_nrb)
              bq[j + PFD] = __builtin_nontemporal_load(
                  (const u32x4_t*)(a.base + (size_t)(ROWREG ? lr[j + PFD].info.rk : n_info[n2].rk) * V + tg));
          }
        }
        const RowInfo info = ROWREG ? lr[j].info : n_info[n];
        const f32x4_t c0 = cb0[j], c1 = cb1[j];
        const bool valid = n < rows;
        const bool active = valid && tok_ok;
        const bool noisy = !(info.T == 0.0f);
        const bool top2 = noisy && !exact_mode;
        uint32_t bw[4];
        bw[0] = pack_bf16(c0[0], c0[1]);
        bw[1] = pack_bf16(c0[2], c0[3]);
        bw[2] = pack_bf16(c1[0], c1[1]);
        bw[3] = pack_bf16(c1[2], c1[3]);
        if (bias_mode) {
          if (active)
            *(uint4*)(a.bias_out + (size_t)n_row[n] * V + tg) = make_uint4(bw[0], bw[1], bw[2], bw[3]);
        } else {
          const u32x4_t bv = bq[j];
          // this slot is free again: the next slab's logits for the same row
          if (MARKOV_XSLAB && j < PFD) {
            bq[j] = (u32x4_t){0u, 0u, 0u, 0u};
            if (valid && tokn_ok && (my_nrb > PFD || j + PFD >= my_nrb))
              bq[j] = __builtin_nontemporal_load((const u32x4_t*)(a.base + (size_t)info.rk * V + tgn));
          }
          // logits: bf16 add (one binary32 add, rounded), multiplier, soft cap
          const uint32_t bwd[4] = {bv.x, bv.y, bv.z, bv.w};
          float l[8];
          uint32_t cw[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            cw[q] = pack_bf16(bf_lo(bwd[q]) + bf_lo(bw[q]), bf_hi(bwd[q]) + bf_hi(bw[q]));
          if (a.has_cap) {
            float z[8];
            float zmax = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              z[2 * q] = (mult * bf_lo(cw[q])) * inv_cap;
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
            for (int q = 0; q < 4; ++q)
              cw[q] = pack_bf16(mult * bf_lo(cw[q]), mult * bf_hi(cw[q]));
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            l[2 * q] = bf_lo(cw[q]);
            l[2 * q + 1] = bf_hi(cw[q]);
          }
          if (active)
            __builtin_nontemporal_store((u32x4_t){cw[0], cw[1], cw[2], cw[3]},
                                        (u32x4_t*)(a.cache + (size_t)info.rk * V + tg));

          if (__any(active && top2)) {
            if (active && top2) {
              bool special = false;
              float v1 = lr[j].v1, v2 = lr[j].v2;
              int eb = -1;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t h = mm_finish(info.prefix, kw[e]);
                const float ka = key_fast(l[e], info.rcp, h);
                const bool bad = !(fabsf(ka) < 1e37f);
                special = special || bad;
                const float hx = bad ? -INFINITY : upper_of(ka);
                // elements arrive in rising id: a tie keeps the earlier as top
                eb = hx > v1 ? e : eb;
                v2 = __builtin_amdgcn_fmed3f(v1, v2, hx);
                v1 = fmaxf(v1, hx);
              }
              lr[j].v1 = v1;
              lr[j].v2 = v2;
              if (eb >= 0) {
                lr[j].id1 = tg + eb;
                lr[j].l1 = pick8(l, eb);
              }
              if (special) atomicAdd(&sp_cnt[n], 1);
            }
          }
          // keep each row block's live ranges to itself
          if (__any(active && !top2)) {
            if (active && !top2) {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                float key = l[e];
                if (noisy) key = key_exact(l[e], info.T, mm_finish(info.prefix, kw[e]));
                if (before(key, tg + e, lr[j].v1, lr[j].id1)) {
                  lr[j].v1 = key;
                  lr[j].id1 = tg + e;
                }
              }
            }
          }
        }
        if (MRB >= 8) __builtin_amdgcn_sched_barrier(0);
      }
      if (!a_out && nxt < a.nslabs)
        load_w2_tile<KB>(a.w2, V, R, nxt * SLAB + wt * TOK_PER_WAVE, m, g, kzero, A0, A1);
    }
  }
  if (bias_mode) return;

  // 3. each row's state: this lane's, merged over the row's 4 lanes, stored
  //    per token wave, then merged over the token waves; one exact key for
  //    the top element of a noisy row (its cached logit read back) unless
  //    another element's bound reaches it (or an estimate was not finite),
  //    in which case the row goes to the exact fallback below; then one
  //    packed atomicMax per row.
#pragma unroll
  for (int j = 0; j < MRB; ++j) {
    if (j >= my_nrb) break;
    RowState st = {lr[j].v1, lr[j].v2, lr[j].l1, lr[j].id1};
#pragma unroll
    for (int sh = 16; sh <= 32; sh <<= 1) {
      RowState o;
      o.v1 = __shfl_xor(st.v1, sh);
      o.v2 = __shfl_xor(st.v2, sh);
      o.l1 = __shfl_xor(st.l1, sh);
      o.id1 = __shfl_xor(st.id1, sh);
      if (!(n_info[(wr + j * RG) * 16 + m].T == 0.0f) && !exact_mode) merge_top2(st, o);
      else merge_order(st, o);
    }
    const int n = (wr + j * RG) * 16 + m;
    if (g == 0 && n < rp) {
      st_v1[wt * rp + n] = st.v1;
      st_v2[wt * rp + n] = st.v2;
      st_l[wt * rp + n] = st.l1;
      st_id[wt * rp + n] = st.id1;
    }
  }
  __syncthreads();
  for (int n = tid; n < rows; n += NTH) {
    const float T = n_info[n].T;
    const bool noisy = !(T == 0.0f);
    const bool top2 = noisy && !exact_mode;
    RowState st = {st_v1[n], st_v2[n], st_l[n], st_id[n]};
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const int i = w * rp + n;
      RowState o = {st_v1[i], st_v2[i], st_l[i], st_id[i]};
      if (top2) merge_top2(st, o);
      else merge_order(st, o);
    }
    const int r = n_row[n];
    float key = st.v1;
    if (top2) {
      const bool near = st.id1 != NONE && st.v2 >= lower_of_upper(st.v1);
      if (near || sp_cnt[n] > 0 || mode == MODE_SAMPLE_FALLBACK) {
        fb_list[atomicAdd(&misc[32], 1)] = n;
        continue;
      }
      key = key_exact(st.l1, T, mm_finish(n_info[n].prefix, mm_token_word((uint32_t)st.id1)));
    }
    if (st.id1 != NONE)
      __hip_atomic_fetch_max(slots_cur + r, pack_winner(key, st.id1), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();

  // 4. exact fallback: the whole workgroup re-reads the row's cached logits
  //    over its own slabs and takes every exact key.
  const int nfb = misc[32];
  if (nfb > 0) {
    __builtin_amdgcn_s_waitcnt(0);   // this workgroup's cache stores, re-read below
    __syncthreads();
  }
  float* red_v = st_v1;  // reuse: [NWV] partials
  int* red_i = st_id;
  for (int f = 0; f < nfb; ++f) {
    const int n = fb_list[f];
    const int r = n_row[n];
    const float T = n_info[n].T;
    const uint32_t prefix = n_info[n].prefix;
    float bv = -INFINITY;
    int bi = NONE;
    const int per_wg = ((a.nslabs - blockIdx.x + G - 1) / G) * SLAB;
    for (int i = tid; i < per_wg; i += NTH) {
      const int t = (blockIdx.x + (i / SLAB) * G) * SLAB + (i % SLAB);
      if (t < V) {
        const float l = bf_lo((uint32_t)a.cache[((size_t)r * K + s) * (size_t)V + t]);
        const float key = key_exact(l, T, mm_finish(prefix, mm_token_word((uint32_t)t)));
        if (before(key, t, bv, bi)) {
          bv = key;
          bi = t;
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
    __syncthreads();
    if (lane == 0) {
      red_v[wave] = bv;
      red_i[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < NWV; ++w)
        if (before(red_v[w], red_i[w], bv, bi)) {
          bv = red_v[w];
          bi = red_i[w];
        }
      if (bi != NONE)
        __hip_atomic_fetch_max(slots_cur + r, pack_winner(bv, bi), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// After the last step: its winners become tokens[:, k-1], and all three
// slot buffers are left zeroed for the next call.
__global__ __launch_bounds__(BLOCK) void markov_finish_kernel(unsigned long long* slots, int64_t* tokens,
                                                              int rows, int k) {
  for (int r = threadIdx.x; r < rows; r += BLOCK) {
    const unsigned long long w = slots[(size_t)((k - 1) % 3) * rows + r];
    tokens[(int64_t)r * k + k - 1] = slot_token(w);
    slots[r] = 0ull;
    slots[(size_t)rows + r] = 0ull;
    slots[(size_t)2 * rows + r] = 0ull;
  }
}

// ---------------------------------------------------------------- test kernels

__global__ void debug_gumbel_kernel(const float* logits, const uint32_t* ids, int64_t n, float T,
                                    int64_t seed, int step, int64_t position, float* kx, float* kf,
                                    float* mg) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t h = mm_finish(row_prefix_of(seed, step, position), mm_token_word(ids[i]));
  float l = logits[i];
  const float ka = key_fast(l, 1.0f / T, h);
  kf[i] = ka;
  mg[i] = fast_margin(ka);
  kx[i] = !(T == 0.0f) ? key_exact(l, T, h) : l;
}

__global__ void debug_bf16_kernel(const float* in, uint16_t* out, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = (uint16_t)(pack_bf16(in[i], 0.0f) & 0xffffu);
}

// A plain copy, 16 bytes per lane per iteration over a grid-stride loop:
// the calibration reference for the DRAM byte counters (it reads and writes
// exactly `n16` * 16 bytes).
__global__ __launch_bounds__(256) void markov_copy_kernel(const u32x4_t* __restrict__ src,
                                                          u32x4_t* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

// ---------------------------------------------------------------- host side

typedef void (*StepFn)(StepArgs);

// Row groups per workgroup: when one workgroup's LDS (mostly the
// embeddings) leaves room for a single workgroup per CU, more waves share it
// (two row groups; four where the rank is small enough to keep the w2 tile in
// few registers). MRB: the most row blocks one wave handles.
size_t lds_bytes(int rows, int R);

struct Plan {
  int rg, mrb;
};

Plan plan_of(int rows, int R) {
  const int nrb = (rows + 15) / 16;
  int rg = 1;
  if (lds_bytes(rows, R) > 80 * 1024) rg = 2;
#ifdef MARKOV_FORCE_RG
  if (nrb >= MARKOV_FORCE_RG) rg = MARKOV_FORCE_RG;
#endif
  const int need = (nrb + rg - 1) / rg;
  int mrb = 1;
  while (mrb < need) mrb *= 2;
  return Plan{rg, mrb};
}

template <int KB, bool EX>
StepFn pick_plan(Plan p) {
  if (p.rg == 1) {
    switch (p.mrb) {
      case 1: return markov_step_kernel<KB, 1, 1, EX>;
      case 2: return markov_step_kernel<KB, 1, 2, EX>;
      case 4: return markov_step_kernel<KB, 1, 4, EX>;
      case 8: return markov_step_kernel<KB, 1, 8, EX>;
    }
  } else if (p.rg == 2) {
    switch (p.mrb) {
      case 1: return markov_step_kernel<KB, 2, 1, EX>;
      case 2: return markov_step_kernel<KB, 2, 2, EX>;
      case 4: return markov_step_kernel<KB, 2, 4, EX>;
      case 8: return markov_step_kernel<KB, 2, 8, EX>;
      case 16: return KB <= 2 ? markov_step_kernel<KB <= 2 ? KB : 1, 2, 16, EX> : nullptr;
      case 32: return KB == 1 ? markov_step_kernel<1, 2, 32, EX> : nullptr;
    }
  }
  return nullptr;
}

template <bool EX>
StepFn pick_rank(int R, Plan p) {
  switch (R) {
    case 16:
    case 32: return pick_plan<1, EX>(p);
    case 64: return pick_plan<2, EX>(p);
    case 128: return pick_plan<4, EX>(p);
    case 256: return pick_plan<8, EX>(p);
    case 512: return pick_plan<16, EX>(p);
  }
  return nullptr;
}

StepFn pick_kernel(int R, Plan p, bool exact = false) {
  return exact ? pick_rank<true>(R, p) : pick_rank<false>(R, p);
}

bool pow2_rank(int R) { return R >= 16 && R <= 512 && (R & (R - 1)) == 0; }

// LDS of one workgroup: the embeddings, per-row data (5 words), the waves'
// running row states (4 words each), the special counts and fallback list,
// and a small misc area.
size_t lds_bytes(int rows, int R) {
  size_t rp = (size_t)((rows + 15) & ~15);
  return rp * R * 2 + rp * 6 * 4 + (size_t)4 * rp * 16 + rp * 8 + 64 * 4;
}

constexpr size_t LDS_MAX = 160 * 1024;

int32_t max_rows_of(int32_t R) {
  if (!pow2_rank(R)) return 0;
  int32_t best = 0;
  for (int32_t rows = 16; rows <= ROWS_CAP; rows += 16)
    if ((size_t)rows * R * 2 <= (size_t)LDS_EMB_MAX && lds_bytes(rows, R) <= LDS_MAX &&
        pick_kernel(R, plan_of(rows, R)) != nullptr)
      best = rows;
  return best;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const markov_shape_t* sh, int32_t k) {
  if (!sh) return MARKOV_ERR_NULL;
  if (sh->rows < 1 || sh->vocab < 1 || (sh->vocab & 7) || k < 1) return MARKOV_ERR_SHAPE;
  if (!pow2_rank(sh->rank)) return MARKOV_ERR_RANK;
  if (sh->rows > max_rows_of(sh->rank)) return MARKOV_ERR_ROWS;
  return MARKOV_OK;
}

struct LaunchCache {
  StepFn fn;
  int device;
  size_t lds;
  int grid_cap;
};
LaunchCache g_cache[64];
int g_cache_n = 0;

// Workgroups to launch: as many as are resident at once (occupancy at this
// LDS size times the CU count), never more than there are slabs.
int launch_grid(StepFn fn, size_t lds, int block, int nslabs, int* grid) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MARKOV_ERR_HIP;
  for (int i = 0; i < g_cache_n; ++i) {
    if (g_cache[i].fn == fn && g_cache[i].device == dev && g_cache[i].lds == lds) {
      *grid = nslabs < g_cache[i].grid_cap ? nslabs : g_cache[i].grid_cap;
      return MARKOV_OK;
    }
  }
  if (hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
      hipSuccess)
    return MARKOV_ERR_HIP;
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MARKOV_ERR_HIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)fn, block, lds) != hipSuccess)
    return MARKOV_ERR_HIP;
  if (occ < 1) return MARKOV_ERR_ROWS;
  int cap = cus * occ;
#ifndef MARKOV_GRID_PER_CU
#define MARKOV_GRID_PER_CU 2
#endif
  // at most two resident workgroups per CU: each workgroup's prologue
  // (embedding gather) and per-row atomics are a fixed cost
  if (occ > MARKOV_GRID_PER_CU) cap = cus * MARKOV_GRID_PER_CU;
  if (g_cache_n < 64) g_cache[g_cache_n++] = LaunchCache{fn, dev, lds, cap};
  *grid = nslabs < cap ? nslabs : cap;
  return MARKOV_OK;
}

size_t ws_bytes(int rows) { return (size_t)rows * 8 * 3; }

int launch_steps(int mode, const void* base, const void* w1, const void* w2, const int64_t* prev,
                 const int64_t* seeds, const int64_t* positions, int32_t k, int32_t s_begin,
                 int32_t s_end, const float* temperature, void* cache, int64_t* tokens,
                 void* bias_out, markov_stream_t stream, const markov_shape_t* sh,
                 void* workspace) {
  const Plan plan = plan_of(sh->rows, sh->rank);
  const int rg = plan.rg;
  StepFn fn = pick_kernel(sh->rank, plan, mode == MODE_SAMPLE_EXACT);
  if (!fn) return MARKOV_ERR_ROWS;
  const size_t lds = lds_bytes(sh->rows, sh->rank);
  const int nslabs = (sh->vocab + SLAB - 1) / SLAB;
  const int block = 256 * rg;
  int grid = 0;
  int rc = launch_grid(fn, lds, block, nslabs, &grid);
  if (rc) return rc;
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.base = (const uint16_t*)base;
  a.w1 = (const uint16_t*)w1;
  a.w2 = (const uint16_t*)w2;
  a.prev = prev;
  a.seeds = seeds;
  a.positions = positions;
  a.temperature = temperature;
  a.cache = (uint16_t*)cache;
  a.tokens = tokens;
  a.bias_out = (uint16_t*)bias_out;
  a.slots = (unsigned long long*)workspace;
  a.rows = sh->rows;
  a.V = sh->vocab;
  a.R = sh->rank;
  a.k = k;
  a.nslabs = nslabs;
  a.mode = mode;
  a.mult = sh->mult;
  a.has_cap = sh->softcap > 0.0f;
  a.cap = sh->softcap;
  a.inv_cap = a.has_cap ? 1.0f / sh->softcap : 0.0f;
  for (int s = s_begin; s < s_end; ++s) {
    a.step = s;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(block), lds, (hipStream_t)stream, a);
    if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  }
  if (mode != MODE_BIAS && s_end == k) {
    hipLaunchKernelGGL(markov_finish_kernel, dim3(1), dim3(BLOCK), 0, (hipStream_t)stream,
                       a.slots, tokens, sh->rows, k);
    if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  }
  return MARKOV_OK;
}

int sample_common(int mode, const void* base_logits, const void* w1, const void* w2,
                  const int64_t* prev, const int64_t* seeds, const int64_t* positions, int32_t k,
                  int32_t s_begin, int32_t s_end, const float* temperature, void* cache,
                  int64_t* tokens, markov_stream_t stream, const markov_shape_t* shape,
                  void* workspace, size_t workspace_bytes) {
  int rc = check_shape(shape, k);
  if (rc) return rc;
  if (s_begin < 0 || s_end > k || s_begin >= s_end) return MARKOV_ERR_SHAPE;
  if (!base_logits || !w1 || !w2 || !prev || !seeds || !positions || !temperature || !cache ||
      !tokens || !workspace)
    return MARKOV_ERR_NULL;
  if (!aligned16(base_logits) || !aligned16(w1) || !aligned16(w2) || !aligned16(cache))
    return MARKOV_ERR_ALIGN;
  if (workspace_bytes < ws_bytes(shape->rows)) return MARKOV_ERR_WORKSPACE;
  return launch_steps(mode, base_logits, w1, w2, prev, seeds, positions, k, s_begin, s_end,
                      temperature, cache, tokens, nullptr, stream, shape, workspace);
}

}  // namespace

extern "C" {

int32_t markov_max_rows(int32_t rank) { return max_rows_of(rank); }

size_t markov_workspace_bytes(const markov_shape_t* shape, int32_t k) {
  if (check_shape(shape, k)) return 0;
  return ws_bytes(shape->rows);
}

int markov_workspace_init(void* workspace, size_t bytes, markov_stream_t stream) {
  if (!workspace) return MARKOV_ERR_NULL;
  if (hipMemsetAsync(workspace, 0, bytes, (hipStream_t)stream) != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

const char* markov_why_not(const markov_shape_t* shape, int32_t k) {
  if (!shape) return "no shape";
  if (shape->rows < 1) return "no requests";
  if (k < 1) return "no draft steps";
  if (shape->vocab < 1 || (shape->vocab & 7)) return "vocabulary not a positive multiple of 8";
  if (!pow2_rank(shape->rank)) return "Markov rank not a power of two in [16, 512]";
  if (shape->rows > max_rows_of(shape->rank)) return "more requests than the rank's LDS budget holds";
  return nullptr;
}

int markov_sample_sequential(const void* base_logits, const void* w1, const void* w2,
                             const int64_t* prev, const int64_t* seeds,
                             const int64_t* positions, int32_t k, const float* temperature,
                             void* cache, int64_t* tokens, markov_stream_t stream,
                             const markov_shape_t* shape, void* workspace,
                             size_t workspace_bytes) {
  return sample_common(MODE_SAMPLE, base_logits, w1, w2, prev, seeds, positions, k, 0, k,
                       temperature, cache, tokens, stream, shape, workspace, workspace_bytes);
}

int markov_sample_step(const void* base_logits, const void* w1, const void* w2,
                       const int64_t* prev, const int64_t* seeds, const int64_t* positions,
                       int32_t k, int32_t step, const float* temperature, void* cache,
                       int64_t* tokens, markov_stream_t stream, const markov_shape_t* shape,
                       void* workspace, size_t workspace_bytes) {
  return sample_common(MODE_SAMPLE, base_logits, w1, w2, prev, seeds, positions, k, step,
                       step + 1, temperature, cache, tokens, stream, shape, workspace,
                       workspace_bytes);
}

int markov_debug_sample_fallback(const void* base_logits, const void* w1, const void* w2,
                                 const int64_t* prev, const int64_t* seeds,
                                 const int64_t* positions, int32_t k, const float* temperature,
                                 void* cache, int64_t* tokens, markov_stream_t stream,
                                 const markov_shape_t* shape, void* workspace,
                                 size_t workspace_bytes) {
  return sample_common(MODE_SAMPLE_FALLBACK, base_logits, w1, w2, prev, seeds, positions, k, 0, k,
                       temperature, cache, tokens, stream, shape, workspace, workspace_bytes);
}

int markov_debug_sample_exact(const void* base_logits, const void* w1, const void* w2,
                              const int64_t* prev, const int64_t* seeds,
                              const int64_t* positions, int32_t k, const float* temperature,
                              void* cache, int64_t* tokens, markov_stream_t stream,
                              const markov_shape_t* shape, void* workspace,
                              size_t workspace_bytes) {
  return sample_common(MODE_SAMPLE_EXACT, base_logits, w1, w2, prev, seeds, positions, k, 0, k,
                       temperature, cache, tokens, stream, shape, workspace, workspace_bytes);
}

const char* markov_status_string(int status) {
  switch (status) {
    case MARKOV_OK: return "ok";
    case MARKOV_ERR_NULL: return "a required pointer is NULL";
    case MARKOV_ERR_SHAPE: return "bad shape (rows, vocab or k)";
    case MARKOV_ERR_RANK: return "rank not a power of two in [16, 512]";
    case MARKOV_ERR_ALIGN: return "a bf16 array is not 16-byte aligned";
    case MARKOV_ERR_ROWS: return "more rows than the rank's LDS budget holds";
    case MARKOV_ERR_WORKSPACE: return "workspace too small";
    case MARKOV_ERR_HIP: return "HIP runtime error";
    case MARKOV_ERR_VOCAB: return "vocabulary too large";
  }
  return "unknown status";
}

int markov_debug_bias(const void* w1, const void* w2, const int64_t* tok, void* bias,
                      const markov_shape_t* shape, markov_stream_t stream) {
  int rc = check_shape(shape, 1);
  if (rc) return rc;
  if (!w1 || !w2 || !tok || !bias) return MARKOV_ERR_NULL;
  if (!aligned16(w1) || !aligned16(w2) || !aligned16(bias)) return MARKOV_ERR_ALIGN;
  return launch_steps(MODE_BIAS, nullptr, w1, w2, tok, nullptr, nullptr, 1, 0, 1, nullptr,
                      nullptr, nullptr, bias, stream, shape, nullptr);
}

int markov_debug_gumbel(const float* logits, const uint32_t* ids, int64_t n, float temperature,
                        int64_t seed, int32_t step, int64_t position, float* key_exact_out,
                        float* key_fast_out, float* margin, markov_stream_t stream) {
  if (!logits || !ids || !key_exact_out || !key_fast_out || !margin) return MARKOV_ERR_NULL;
  if (n < 0) return MARKOV_ERR_SHAPE;
  if (n == 0) return MARKOV_OK;
  const int tb = 256;
  const int64_t blocks = (n + tb - 1) / tb;
  debug_gumbel_kernel<<<dim3((unsigned)blocks), tb, 0, (hipStream_t)stream>>>(
      logits, ids, n, temperature, seed, step, position, key_exact_out, key_fast_out, margin);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

int markov_debug_copy(const void* src, void* dst, int64_t bytes, markov_stream_t stream) {
  if (!src || !dst) return MARKOV_ERR_NULL;
  if (bytes < 0 || (bytes & 15)) return MARKOV_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return MARKOV_ERR_ALIGN;
  if (bytes == 0) return MARKOV_OK;
  const int64_t n16 = bytes / 16;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t want = (n16 + 255) / 256;
  const int64_t blocks = want < (int64_t)cus * 8 ? want : (int64_t)cus * 8;
  markov_copy_kernel<<<dim3((unsigned)blocks), 256, 0, (hipStream_t)stream>>>(
      (const u32x4_t*)src, (u32x4_t*)dst, n16);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

int markov_debug_bf16_round(const float* in, uint16_t* out, int64_t n, markov_stream_t stream) {
  if (!in || !out) return MARKOV_ERR_NULL;
  if (n < 0) return MARKOV_ERR_SHAPE;
  if (n == 0) return MARKOV_OK;
  const int tb = 256;
  const int64_t blocks = (n + tb - 1) / tb;
  debug_bf16_kernel<<<dim3((unsigned)blocks), tb, 0, (hipStream_t)stream>>>(in, out, n);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

}  // extern "C"
