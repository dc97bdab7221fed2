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

enum Mode { MODE_SAMPLE = 0, MODE_SAMPLE_EXACT = 1, MODE_BIAS = 2 };

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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
  unsigned long long* slots;
  unsigned int* counter;
  uint16_t* bias_out;
  int rows, V, R, k, step, nslabs;
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
  h = h * 5u + 0xe6546b64u;
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

// Cheap key estimate and its error margin. y = -log(1 - u) by a 4-term
// series below u = 1/16 (truncation < 4e-6 relative), else by the hardware
// log2; the outer log by the hardware log2. |key_fast - key_exact| stays far
// inside `margin` (1e-3 absolute plus 2^-18 relative), which the tests check
// against the exact key over the hash range.
constexpr float LN2F = 0.693147180559945309f;

__device__ __forceinline__ float key_fast(float l, float rcpT, uint32_t h, float* margin) {
  float u = uniform_of(h);
  float ys = u * __builtin_fmaf(u, __builtin_fmaf(u, __builtin_fmaf(u, 0.25f, 1.0f / 3.0f), 0.5f), 1.0f);
  float yl = -LN2F * __builtin_amdgcn_logf(fmaxf(1.0f - u, 0x1p-24f));
  float y = u < 0.0625f ? ys : yl;
  float g = -LN2F * __builtin_amdgcn_logf(y);
  float q = l * rcpT;
  float ka = q + g;
  *margin = 1e-3f + (fabsf(q) + fabsf(ka)) * 0x1p-18f;
  return ka;
}

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

template <int KB, int MODE>
__global__ __launch_bounds__(BLOCK) void markov_step_kernel(StepArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, m = lane & 15;
  const int rows = a.rows, rows_pad = (rows + 15) & ~15, R = a.R, V = a.V, s = a.step;
  const int cpr = R >> 3;                       // 16-byte chunks per embedding row
  const int swz = (cpr < 8 ? cpr : 8) - 1;

  uint16_t* emb = (uint16_t*)lds;
  uint32_t* row_prefix = (uint32_t*)(lds + (size_t)rows_pad * R * 2);
  float* row_T = (float*)(row_prefix + rows_pad);
  float* row_rcp = row_T + rows_pad;
  int* row_src = (int*)(row_rcp + rows_pad);
  float* best_key = (float*)(row_src + rows_pad);  // [NW][rows_pad]
  int* best_id = (int*)(best_key + NW * rows_pad);
  int* flag = best_id + NW * rows_pad;

  // 1. per-row set-up: the token feeding this step, clamped; temperature;
  //    the hash prefix; empty running winners.
  for (int r = tid; r < rows_pad; r += BLOCK) {
    if (r < rows) {
      int64_t t = (MODE == MODE_BIAS || s == 0) ? a.prev[r] : a.tokens[(int64_t)r * a.k + s - 1];
      uint64_t ut = (uint64_t)t, last = (uint64_t)(V - 1);
      row_src[r] = (int)(ut < last ? ut : last);
      if (MODE != MODE_BIAS) {
        float T = a.temperature[r];
        row_T[r] = T;
        row_rcp[r] = 1.0f / T;
        row_prefix[r] = row_prefix_of(a.seeds[r], s, a.positions[(int64_t)r * a.k + s]);
      }
    } else {
      row_src[r] = -1;
      row_T[r] = 0.0f;
      row_rcp[r] = 0.0f;
      row_prefix[r] = 0u;
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      best_key[w * rows_pad + r] = -INFINITY;
      best_id[w * rows_pad + r] = NONE;
    }
  }
  __syncthreads();

  // 2. gather the rows' embeddings into LDS (padding rows are zero).
  for (int c = tid; c < rows_pad * cpr; c += BLOCK) {
    int n = c / cpr, ch = c - n * cpr;
    int src = row_src[n];
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (src >= 0) v = ld16(a.w1 + (size_t)src * R + ch * 8);
    *(uint4*)(emb + (size_t)n * R + ((ch ^ (n & swz)) * 8)) = v;
  }
  __syncthreads();

  const int nrb = rows_pad >> 4;
  const bool kzero = (R == 16) && (g >= 2);     // rank 16 fills half a K=32 block

  for (int slab = blockIdx.x; slab < a.nslabs; slab += gridDim.x) {
    const int tok0 = slab * SLAB + wave * TOK_PER_WAVE;
    if (tok0 >= V) continue;                    // wave-uniform: past the vocabulary

    // A operands: M-tile 0 row mm holds token tok0 + 8(mm/4) + mm%4, M-tile 1
    // the same + 4; K chunk (4i + g) of the row feeds k-block i, lane group g.
    bf16x8_t A0[KB], A1[KB];
    {
      const int t0 = tok0 + 8 * (m >> 2) + (m & 3);
      const int ta = t0 < V ? t0 : V - 1, tb = t0 + 4 < V ? t0 + 4 : V - 1;
      const uint16_t* pa = a.w2 + (size_t)ta * R;
      const uint16_t* pb = a.w2 + (size_t)tb * R;
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
    const int tg = tok0 + 8 * g;                // this lane's 8 tokens: tg .. tg+7
    const bool tok_ok = tg < V;
    uint32_t kw[8];
    if (MODE != MODE_BIAS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) kw[e] = mm_token_word((uint32_t)(tg + e));
    }

    for (int rb = 0; rb < nrb; ++rb) {
      const int n = rb * 16 + m;                // this lane's row
      f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
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
      const bool active = (n < rows) && tok_ok;
      // bias rounded once to bf16, two per word, tokens tg .. tg+7
      uint32_t bw[4];
      bw[0] = pack_bf16(c0[0], c0[1]);
      bw[1] = pack_bf16(c0[2], c0[3]);
      bw[2] = pack_bf16(c1[0], c1[1]);
      bw[3] = pack_bf16(c1[2], c1[3]);

      if (MODE == MODE_BIAS) {
        if (active) *(uint4*)(a.bias_out + (size_t)n * V + tg) = make_uint4(bw[0], bw[1], bw[2], bw[3]);
        continue;
      }

      const float T = row_T[n], rcpT = row_rcp[n];
      const uint32_t prefix = row_prefix[n];
      const bool noisy = !(T == 0.0f);
      float l[8];
      uint32_t h[8];
      float lo_max = -INFINITY;
      float lane_key = -INFINITY;
      int lane_id = NONE;
      uint32_t cand = 0u;
      float hi_e[8];
      if (active) {
        const size_t off = ((size_t)n * a.k + s) * (size_t)V + tg;
        const uint4 bv = ld16(a.base + off);
        const uint32_t bwd[4] = {bv.x, bv.y, bv.z, bv.w};
        uint32_t cw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // bf16 add: one binary32 add, rounded to bf16
          uint32_t xp = pack_bf16(bf_lo(bwd[q]) + bf_lo(bw[q]), bf_hi(bwd[q]) + bf_hi(bw[q]));
          float y0 = a.mult * bf_lo(xp), y1 = a.mult * bf_hi(xp);
          if (a.has_cap) {
            y0 = a.cap * tanhf(y0 * a.inv_cap);
            y1 = a.cap * tanhf(y1 * a.inv_cap);
          }
          cw[q] = pack_bf16(y0, y1);
          l[2 * q] = bf_lo(cw[q]);
          l[2 * q + 1] = bf_hi(cw[q]);
        }
        *(uint4*)(a.cache + off) = make_uint4(cw[0], cw[1], cw[2], cw[3]);

        if (!noisy) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (before(l[e], tg + e, lane_key, lane_id)) { lane_key = l[e]; lane_id = tg + e; }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            h[e] = mm_finish(prefix, kw[e]);
            if (MODE == MODE_SAMPLE_EXACT) {
              hi_e[e] = __builtin_nanf("");     // every element is a candidate
            } else {
              float mg;
              float ka = key_fast(l[e], rcpT, h[e], &mg);
              if (__builtin_isfinite(ka) && fabsf(ka) < 1e37f) {
                lo_max = fmaxf(lo_max, ka - mg);
                hi_e[e] = ka + mg;
              } else {
                hi_e[e] = __builtin_nanf("");   // always a candidate
              }
            }
          }
        }
      }
      // the row's best lower bound over its 4 lanes (32 tokens)
      lo_max = fmaxf(lo_max, __shfl_xor(lo_max, 16));
      lo_max = fmaxf(lo_max, __shfl_xor(lo_max, 32));
      const float Bk = best_key[wave * rows_pad + n];
      const int Bi = best_id[wave * rows_pad + n];
      if (active && noisy) {
        const bool b_none = (Bi == NONE), b_nan = __builtin_isnan(Bk);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bool c;
          if (__builtin_isnan(hi_e[e])) c = b_none || !b_nan;
          else c = hi_e[e] >= lo_max && (b_none || (!b_nan && hi_e[e] > Bk));
          cand |= (c ? 1u : 0u) << e;
        }
      }
      // exact keys of the candidates, one per lane per round
      while (__any(cand != 0u)) {
        if (cand != 0u) {
          const int e = __builtin_ctz(cand);
          cand &= cand - 1u;
          const float le = pick8(l, e);
          const uint32_t he = pick8(h, e);
          const float kx = key_exact(le, T, he);
          if (before(kx, tg + e, lane_key, lane_id)) { lane_key = kx; lane_id = tg + e; }
        }
      }
      // the row's winner over its 4 lanes, then into the wave's running best
#pragma unroll
      for (int sh = 16; sh <= 32; sh <<= 1) {
        float ok = __shfl_xor(lane_key, sh);
        int oi = __shfl_xor(lane_id, sh);
        if (before(ok, oi, lane_key, lane_id)) { lane_key = ok; lane_id = oi; }
      }
      if (g == 0 && n < rows && before(lane_key, lane_id, Bk, Bi)) {
        best_key[wave * rows_pad + n] = lane_key;
        best_id[wave * rows_pad + n] = lane_id;
      }
    }
  }
  if (MODE == MODE_BIAS) return;

  // 3. this workgroup's winner per row -> one packed atomicMax per row.
  __syncthreads();
  for (int r = tid; r < rows; r += BLOCK) {
    float bk = best_key[r];
    int bi = best_id[r];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      float k2 = best_key[w * rows_pad + r];
      int i2 = best_id[w * rows_pad + r];
      if (before(k2, i2, bk, bi)) { bk = k2; bi = i2; }
    }
    if (bi != NONE)
      __hip_atomic_fetch_max(a.slots + r, pack_winner(bk, bi), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
  // 4. arrival: release this workgroup's maxima; the last to arrive acquires
  //    them all, writes the step's tokens and re-zeroes slots and counter.
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    unsigned int ticket = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    *flag = (ticket == gridDim.x - 1) ? 1 : 0;
  }
  __syncthreads();
  if (*flag) {
    __threadfence();
    for (int r = tid; r < rows; r += BLOCK) {
      unsigned long long w = __hip_atomic_load(a.slots + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.tokens[(int64_t)r * a.k + s] = (int64_t)(uint32_t)(~(uint32_t)w);
      __hip_atomic_store(a.slots + r, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  float margin;
  kf[i] = key_fast(l, 1.0f / T, h, &margin);
  mg[i] = margin;
  kx[i] = !(T == 0.0f) ? key_exact(l, T, h) : l;
}

__global__ void debug_bf16_kernel(const float* in, uint16_t* out, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = (uint16_t)(pack_bf16(in[i], 0.0f) & 0xffffu);
}

// ---------------------------------------------------------------- host side

typedef void (*StepFn)(StepArgs);

template <int MODE>
StepFn pick_kernel(int R) {
  switch (R) {
    case 16:
    case 32: return markov_step_kernel<1, MODE>;
    case 64: return markov_step_kernel<2, MODE>;
    case 128: return markov_step_kernel<4, MODE>;
    case 256: return markov_step_kernel<8, MODE>;
    case 512: return markov_step_kernel<16, MODE>;
  }
  return nullptr;
}

bool pow2_rank(int R) { return R >= 16 && R <= 512 && (R & (R - 1)) == 0; }

int32_t max_rows_of(int32_t R) {
  if (!pow2_rank(R)) return 0;
  int32_t by_lds = LDS_EMB_MAX / (R * 2);
  return by_lds < ROWS_CAP ? by_lds : ROWS_CAP;
}

size_t lds_bytes(int rows, int R) {
  size_t rp = (size_t)((rows + 15) & ~15);
  return rp * R * 2 + rp * 4 * 4 + (size_t)NW * rp * 8 + 16;
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
LaunchCache g_cache[32];
int g_cache_n = 0;

// Workgroups to launch: as many as are resident at once (occupancy at this
// LDS size times the CU count), never more than there are slabs.
int launch_grid(StepFn fn, size_t lds, int nslabs, int* grid) {
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
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)fn, BLOCK, lds) != hipSuccess)
    return MARKOV_ERR_HIP;
  if (occ < 1) return MARKOV_ERR_ROWS;
  int cap = cus * occ;
  if (g_cache_n < 32) g_cache[g_cache_n++] = LaunchCache{fn, dev, lds, cap};
  *grid = nslabs < cap ? nslabs : cap;
  return MARKOV_OK;
}

struct Workspace {
  unsigned long long* slots;
  unsigned int* counter;
};

size_t ws_bytes(int rows) { return (size_t)rows * 8 + 256; }

Workspace ws_layout(void* w, int rows) {
  Workspace out;
  out.slots = (unsigned long long*)w;
  out.counter = (unsigned int*)((unsigned char*)w + (size_t)rows * 8);
  return out;
}

int launch_steps(int mode, const void* base, const void* w1, const void* w2, const int64_t* prev,
                 const int64_t* seeds, const int64_t* positions, int32_t k, int32_t s_begin,
                 int32_t s_end, const float* temperature, void* cache, int64_t* tokens,
                 void* bias_out, markov_stream_t stream, const markov_shape_t* sh,
                 void* workspace) {
  StepFn fn = mode == MODE_SAMPLE ? pick_kernel<MODE_SAMPLE>(sh->rank)
            : mode == MODE_SAMPLE_EXACT ? pick_kernel<MODE_SAMPLE_EXACT>(sh->rank)
                                        : pick_kernel<MODE_BIAS>(sh->rank);
  if (!fn) return MARKOV_ERR_RANK;
  const size_t lds = lds_bytes(sh->rows, sh->rank);
  const int nslabs = (sh->vocab + SLAB - 1) / SLAB;
  int grid = 0;
  int rc = launch_grid(fn, lds, nslabs, &grid);
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
  if (workspace) {
    Workspace ws = ws_layout(workspace, sh->rows);
    a.slots = ws.slots;
    a.counter = ws.counter;
  }
  a.rows = sh->rows;
  a.V = sh->vocab;
  a.R = sh->rank;
  a.k = k;
  a.nslabs = nslabs;
  a.mult = sh->mult;
  a.has_cap = sh->softcap > 0.0f;
  a.cap = sh->softcap;
  a.inv_cap = a.has_cap ? 1.0f / sh->softcap : 0.0f;
  for (int s = s_begin; s < s_end; ++s) {
    a.step = s;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(BLOCK), lds, (hipStream_t)stream, a);
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
