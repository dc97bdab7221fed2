// MI355X (gfx950) DSpark sequential Markov draft-sampling step: host side.
//
// The step kernel itself is in step_kernel.h (compiled per rank class in
// step_kb*.hip); this file holds the host-built tables, the launch code, the
// test-only kernels and the C ABI of include/markov.h.

#include "step_kernel.h"

namespace {

// ---------------------------------------------------------------- test kernels

__global__ void debug_gumbel_kernel(const float* logits, const uint32_t* ids, int64_t n, float T,
                                    int64_t seed, int step, int64_t position, const float2* gtable,
                                    float* kx, float* ku) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t h = mm_finish(row_prefix_of(seed, step, position), mm_token_word(ids[i]));
  float l = logits[i];
  ku[i] = key_upper(l, 1.0f / T, noise_bound<true>(gtable, h));
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

// The noise bound table (see gt_index): for each bucket, the chord of the
// noise -lb(h) between the bucket's first and last h, as a line in float(h),
// then raised until it lies on or above the noise everywhere in the bucket,
// checked on a grid of at most GT_GRID intervals in the kernel's own binary32
// evaluation (every hash of a bucket narrower than that), and by 1e-5.
float2 g_table[GT_PAD];
float g_ctable[GTC_PAD];   // a constant bound per bucket
std::once_flag g_table_once;   // the tables are built once per process, by whichever thread comes first

float up_to_float(double x) {
  float f = (float)x;
  if ((double)f < x) f = nextafterf(f, INFINITY);
  return f;
}

// the smallest h whose bucket is b or above (b >= 1): below 2^24 every
// integer is exact; above it, h reaches at least the midpoint between F's
// predecessor and F (F's mantissa is even, so the midpoint rounds up to F)
uint64_t bucket_first_h(int b) {
  if (b >= GT_N) return (uint64_t)1 << 32;
  if (b == 0) return 0;
  const uint32_t fb = (uint32_t)(b + GT_BASE) << 17;
  float F;
  memcpy(&F, &fb, 4);
  const double Fd = (double)F;
  const double h = Fd <= 0x1p24 ? ceil(Fd) : floor(0.5 * ((double)nextafterf(F, 0.0f) + Fd));
  return (uint64_t)h;
}

float line_at(float2 ab, uint32_t h) { return fmaf(ab.y, (float)h, ab.x); }

void build_table_once() {
  std::vector<float> n((size_t)GT_GRID + 1);
  std::vector<uint32_t> hs((size_t)GT_GRID + 1);
  for (int b = 0; b < GT_N; ++b) {
    const uint64_t h0 = bucket_first_h(b), h1 = bucket_first_h(b + 1);
    if (h1 <= h0) {   // no h falls in this bucket
      g_table[b] = make_float2(0.0f, 0.0f);
      g_ctable[b] = 0.0f;
      continue;
    }
    const uint64_t span = h1 - 1 - h0;
    const int M = span < (uint64_t)GT_GRID ? (int)span : GT_GRID;
    for (int i = 0; i <= M; ++i) {
      hs[i] = (uint32_t)(h0 + (M ? span * (uint64_t)i / (uint64_t)M : 0));
      n[i] = -noise_lb(hs[i]);
    }
    double B = 0.0;
    const double f0 = (double)(float)hs[0], f1 = (double)(float)hs[M];
    if (M > 0 && f1 > f0) B = ((double)n[M] - (double)n[0]) / (f1 - f0);
    if (B > 0.0) B = 0.0;   // the line must fall with h
    float2 ab = make_float2(0.0f, (float)B);
    if (ab.y > 0.0f) ab.y = 0.0f;
    ab.x = up_to_float((double)n[0] - (double)ab.y * f0);
    // shortfall: noise at a grid point above the line at the next one (a
    // hash strictly between them has no more noise and no less line), or at
    // the point itself where the next point is the next hash
    for (int pass = 0; pass < 4; ++pass) {
      double short_by = (double)n[M] - (double)line_at(ab, hs[M]);
      for (int i = 0; i < M; ++i) {
        const uint32_t hl = hs[i + 1] == hs[i] + 1 ? hs[i] : hs[i + 1];
        const double d = (double)n[i] - (double)line_at(ab, hl);
        if (d > short_by) short_by = d;
      }
      if (pass > 0 && short_by <= -1e-5) break;
      ab.x = up_to_float((double)ab.x + (short_by > 0.0 ? short_by : 0.0) + 1e-5);
    }
    g_table[b] = ab;
    double top = (double)n[0];
    for (int i = 1; i <= M; ++i) top = (double)n[i] > top ? (double)n[i] : top;
    g_ctable[b] = up_to_float(top + 1e-5);
  }
  for (int b = GT_N; b < GT_PAD; ++b) g_table[b] = make_float2(0.0f, 0.0f);   // unused
  for (int b = GT_N; b < GTC_PAD; ++b) g_ctable[b] = 0.0f;
}

void build_table() { std::call_once(g_table_once, build_table_once); }

// ---- the transform table, host side: c(x) for x = +0 .. the largest bf16
// pattern below the sign bit, with the same operations the kernel's own
// evaluation takes, each rounded once; tanh correctly rounded to binary32
// (binary64 tanh, re-evaluated in x87 extended precision when the binary64
// value lies within a few of its ulps of a binary32 rounding boundary).
uint16_t bf16_rne_host(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);   // NaN stays NaN
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

float tanh_cr_host(float z) {
  const double t = tanh((double)z);
  float f = (float)t;
  if (!(t == t)) return f;
  const float g = (double)f < t ? nextafterf(f, INFINITY) : nextafterf(f, -INFINITY);
  const double mid = 0.5 * ((double)f + (double)g);
  if (fabs(t - mid) <= 16.0 * 0x1p-53 * fabs(t)) f = (float)tanhl((long double)z);
  return f;
}

uint16_t transform_host(uint16_t xb, float mult, float cap) {
  const uint32_t xu = (uint32_t)xb << 16;
  float x;
  memcpy(&x, &xu, 4);
  const float inv_cap = 1.0f / cap;
  const float y = mult * x;
  const float z = y * inv_cap;
  const float w = cap * tanh_cr_host(z);
  return bf16_rne_host(w);
}

// Built tables, kept for the life of the process (an enqueued copy may still
// read one after the call that asked for it has returned).
struct TransformTable {
  uint32_t mult_bits, cap_bits;
  uint32_t data[(TT_HEAD + TT_BYTES) / 4];
};
std::mutex g_tt_mutex;
std::vector<TransformTable*> g_tt;

const TransformTable* transform_table(float mult, float cap) {
  uint32_t mb, cb;
  memcpy(&mb, &mult, 4);
  memcpy(&cb, &cap, 4);
  std::lock_guard<std::mutex> lock(g_tt_mutex);
  for (const TransformTable* t : g_tt)
    if (t->mult_bits == mb && t->cap_bits == cb) return t;
  TransformTable* t = new TransformTable;
  t->mult_bits = mb;
  t->cap_bits = cb;
  memset(t->data, 0, sizeof(t->data));
  t->data[0] = TT_MAGIC;
  t->data[1] = mb;
  t->data[2] = cb;
  uint16_t* e = (uint16_t*)((unsigned char*)t->data + TT_HEAD);
  for (uint32_t i = 0; i < TT_BYTES / 2; ++i) e[i] = transform_host((uint16_t)i, mult, cap);
  g_tt.push_back(t);
  return t;
}

struct Plan {
  int rg, mrb;
};

// Row blocks: each wave handles all of them (up to 8), else the two waves
// of a SIMD split them (row groups; past 16 row blocks a wave keeps 16 and
// spills registers).
Plan plan_of(int rows) {
  const int nrb = (rows + 15) / 16;
  const int rg = nrb > MRB_MAX ? 2 : 1;
  const int need = (nrb + rg - 1) / rg;
  int mrb = 1;
  while (mrb < need) mrb *= 2;
  return Plan{rg, mrb};
}

// The step kernel of a rank, plan and variant (V_SAMPLE, V_EXACT, V_GREEDY).
StepFn pick_kernel(int R, Plan p, int var = V_SAMPLE) {
  const int kb = R == 16 ? 1 : R / 32;
#define MARKOV_PICK(KB, VAR) \
  if (kb == KB && var == VAR) return markov_impl::step_kernel_kb##KB##_v##VAR(p.rg, p.mrb);
  MARKOV_STEP_INSTANCES(MARKOV_PICK)
#undef MARKOV_PICK
  return nullptr;
}

bool pow2_rank(int R) { return R >= 16 && R <= 512 && (R & (R - 1)) == 0; }

size_t lds_bytes(int rows, int R) { return lds_total((rows + 15) & ~15, R); }

int32_t max_rows_of(int32_t R) {
  if (!pow2_rank(R)) return 0;
  int32_t best = 0;
  for (int32_t rows = 16; rows <= ROWS_CAP; rows += 16)
    if (lds_bytes(rows, R) <= LDS_MAX && pick_kernel(R, plan_of(rows)) != nullptr) best = rows;
  return best;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const markov_shape_t* sh, int32_t k) {
  if (!sh) return MARKOV_ERR_NULL;
  if (sh->rows < 1 || sh->vocab < 1 || (sh->vocab & 7) || k < 1) return MARKOV_ERR_SHAPE;
  if (sh->vocab > MARKOV_MAX_VOCAB) return MARKOV_ERR_VOCAB;
  if (!pow2_rank(sh->rank)) return MARKOV_ERR_RANK;
  if (sh->rows > max_rows_of(sh->rank)) return MARKOV_ERR_ROWS;
  return MARKOV_OK;
}

// Per (kernel, device): its dynamic-LDS limit raised to the largest any plan
// uses (the attribute holds one value per kernel, so it is set once, to the
// maximum, rather than per launch size), and the device's CU count.
struct LaunchCache {
  StepFn fn;
  int device;
  int cus;
};
constexpr int LAUNCH_CACHE = 512;
LaunchCache g_cache[LAUNCH_CACHE];
int g_cache_n = 0;
std::mutex g_cache_mutex;   // host threads may launch concurrently

// Workgroups to launch: one per CU (the kernel is sized for one resident
// 8-wave workgroup), never more than there are slabs (a workgroup's second
// waves take slab blockIdx + grid, if there is one).
int launch_grid(StepFn fn, size_t lds, int nslabs, int* grid) {
  if (lds > LDS_MAX) return MARKOV_ERR_ROWS;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MARKOV_ERR_HIP;
  int cus = 0;
  std::lock_guard<std::mutex> lock(g_cache_mutex);
  for (int i = 0; i < g_cache_n; ++i)
    if (g_cache[i].fn == fn && g_cache[i].device == dev) cus = g_cache[i].cus;
  if (cus == 0) {
    if (hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)LDS_MAX) != hipSuccess)
      return MARKOV_ERR_HIP;
    int occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return MARKOV_ERR_HIP;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)fn, NTH, LDS_MAX) !=
        hipSuccess)
      return MARKOV_ERR_HIP;
    if (occ < 1 || cus < 1) return MARKOV_ERR_ROWS;
    if (g_cache_n < LAUNCH_CACHE) g_cache[g_cache_n++] = LaunchCache{fn, dev, cus};
  }
  *grid = nslabs < cus ? nslabs : cus;
  return MARKOV_OK;
}

size_t ws_bytes(int rows) { return (size_t)WS_SLOTS + (size_t)rows * 8 * 3 * SG; }

// One call's arguments: the mode (runtime) and variant (compile time) of the
// kernel, the caller's buffers and the steps to launch.
struct Call {
  int mode = MODE_SAMPLE, var = V_SAMPLE;
  const void *base = nullptr, *w1 = nullptr, *w2 = nullptr;
  const int64_t *prev = nullptr, *seeds = nullptr, *positions = nullptr;
  const float* temperature = nullptr;
  void* cache = nullptr;
  int64_t* tokens = nullptr;
  unsigned long long* winners = nullptr;
  const uint8_t* w2q = nullptr;               // E4M3 w2 (with var & V_W8)
  const uint16_t* w2s = nullptr;
  unsigned long long* packets = nullptr;      // a vocabulary shard's output
  int64_t feed_stride = 1;
  int32_t id_offset = 0, vocab_total = 0;     // 0: the shape's vocab
  void* bias_out = nullptr;
  int32_t k = 1, s_begin = 0, s_end = 1;
};

int launch_steps(const Call& c, markov_stream_t stream, const markov_shape_t* sh, void* workspace) {
  const Plan plan = plan_of(sh->rows);
  StepFn fn = pick_kernel(sh->rank, plan, c.var);
  if (!fn) return MARKOV_ERR_ROWS;
  const bool greedy = (c.var & V_GREEDY) != 0;
  const int rp = (sh->rows + 15) & ~15;
  // (the kernel reads the table's stamp from the workspace whenever this is set)
  const bool tt_layout = c.mode != MODE_BIAS && workspace != nullptr && sh->softcap > 0.0f &&
                         plan.rg == 1 && tt_fits(rp, sh->rank, greedy);
  size_t lds = (tt_layout ? TT_BYTES : 0) + lds_total(rp, sh->rank, greedy);
  const int nslabs = (sh->vocab + SLAB - 1) / SLAB;
  int grid = 0;
  int rc = launch_grid(fn, lds, nslabs, &grid);
  if (rc) return rc;
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.base = (const uint16_t*)c.base;
  a.w1 = (const uint16_t*)c.w1;
  a.w2 = (const uint16_t*)c.w2;
  a.prev = c.prev;
  a.seeds = c.seeds;
  a.positions = c.positions;
  a.temperature = c.temperature;
  a.cache = (uint16_t*)c.cache;
  a.tokens = c.tokens;
  a.winners = c.winners;
  a.w2q = c.w2q;
  a.w2s = c.w2s;
  a.packets = c.packets;
  a.feed_stride = c.feed_stride;
  a.id_offset = c.id_offset;
  a.V_total = c.vocab_total > 0 ? c.vocab_total : sh->vocab;
  a.bias_out = (uint16_t*)c.bias_out;
  if (workspace) {
    a.gtable = (const float*)workspace;
    a.ttable = (const uint32_t*)((unsigned char*)workspace + WS_TT);
    a.slots = (unsigned long long*)((unsigned char*)workspace + WS_SLOTS);
    a.ticket = (unsigned int*)((unsigned char*)workspace + WS_TICKET);
  }
  a.tt_layout = tt_layout ? 1 : 0;
  a.rows = sh->rows;
  a.V = sh->vocab;
  a.R = sh->rank;
  a.k = c.k;
  a.nslabs = nslabs;
  a.mode = c.mode;
  a.mult = sh->mult;
  a.has_cap = sh->softcap > 0.0f;
  a.cap = sh->softcap;
  a.inv_cap = a.has_cap ? 1.0f / sh->softcap : 0.0f;
  a.inf = INFINITY;
  for (int s = c.s_begin; s < c.s_end; ++s) {
    a.step = s;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NTH), lds, (hipStream_t)stream, a);
    if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  }
  return MARKOV_OK;
}

int sample_common(int mode, const void* base_logits, const void* w1, const void* w2,
                  const int64_t* prev, const int64_t* seeds, const int64_t* positions, int32_t k,
                  int32_t s_begin, int32_t s_end, const float* temperature, void* cache,
                  int64_t* tokens, markov_stream_t stream, const markov_shape_t* shape,
                  void* workspace, size_t workspace_bytes, const uint8_t* w2q = nullptr,
                  const uint16_t* w2s = nullptr) {
  int rc = check_shape(shape, k);
  if (rc) return rc;
  if (s_begin < 0 || s_end > k || s_begin >= s_end) return MARKOV_ERR_SHAPE;
  const bool w8 = w2q != nullptr || w2s != nullptr;
  if (!base_logits || !w1 || (!w8 && !w2) || (w8 && (!w2q || !w2s)) || !prev || !seeds ||
      !positions || !temperature || !cache || !tokens || !workspace)
    return MARKOV_ERR_NULL;
  if (!aligned16(base_logits) || !aligned16(w1) || (!w8 && !aligned16(w2)) || !aligned16(cache) ||
      !aligned16(workspace) || (w8 && (!aligned16(w2q) || !aligned16(w2s))))
    return MARKOV_ERR_ALIGN;
  if (workspace_bytes < ws_bytes(shape->rows)) return MARKOV_ERR_WORKSPACE;
  Call c;
  c.mode = mode;
  c.var = (mode == MODE_SAMPLE_EXACT ? V_EXACT : V_SAMPLE) | (w8 ? V_W8 : 0);
  c.w2q = w2q;
  c.w2s = w2s;
  c.base = base_logits;
  c.w1 = w1;
  c.w2 = w2;
  c.prev = prev;
  c.seeds = seeds;
  c.positions = positions;
  c.temperature = temperature;
  c.cache = cache;
  c.tokens = tokens;
  c.k = k;
  c.s_begin = s_begin;
  c.s_end = s_end;
  return launch_steps(c, stream, shape, workspace);
}

int greedy_common(const void* base_logits, const void* w1, const void* w2, const int64_t* prev,
                  int32_t k, int32_t s_begin, int32_t s_end, void* cache, int64_t* tokens,
                  unsigned long long* winners, markov_stream_t stream,
                  const markov_shape_t* shape, void* workspace, size_t workspace_bytes,
                  const uint8_t* w2q = nullptr, const uint16_t* w2s = nullptr) {
  int rc = check_shape(shape, k);
  if (rc) return rc;
  if (s_begin < 0 || s_end > k || s_begin >= s_end) return MARKOV_ERR_SHAPE;
  const bool w8 = w2q != nullptr || w2s != nullptr;
  if (!base_logits || !w1 || (!w8 && !w2) || (w8 && (!w2q || !w2s)) || !prev || !tokens ||
      !workspace)
    return MARKOV_ERR_NULL;
  if (!aligned16(base_logits) || !aligned16(w1) || (!w8 && !aligned16(w2)) ||
      !aligned16(workspace) || (cache && !aligned16(cache)) ||
      (w8 && (!aligned16(w2q) || !aligned16(w2s))))
    return MARKOV_ERR_ALIGN;
  if (workspace_bytes < ws_bytes(shape->rows)) return MARKOV_ERR_WORKSPACE;
  Call c;
  c.mode = MODE_GREEDY;
  c.var = V_GREEDY | (w8 ? V_W8 : 0);
  c.w2q = w2q;
  c.w2s = w2s;
  c.base = base_logits;
  c.w1 = w1;
  c.w2 = w2;
  c.prev = prev;
  c.cache = cache;
  c.tokens = tokens;
  c.winners = winners;
  c.k = k;
  c.s_begin = s_begin;
  c.s_end = s_end;
  return launch_steps(c, stream, shape, workspace);
}

// ---- E4M3 w2 (the Edge-LLM page's `dsparkQuantizeMarkovW2Fp8`)

// E4M3 code of x: nearest, ties to even, saturating at +-448, NaN to the NaN
// code of its sign. Integer rounding on x's bits: at or above 2^-6 the top 3
// fraction bits are kept (a carry moves into the exponent), the exponent
// rebiased from 127 to 7; below, the subnormal m 2^-9 with m = RN(|x| 2^9)
// (m = 8 is the smallest normal, code 8).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x), sgn = (u >> 24) & 0x80u, a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sgn | 0x7fu;
  if (a >= 0x43e00000u) return sgn | 0x7eu;                     // |x| >= 448
  if (a < 0x3c800000u) return sgn | (uint32_t)rintf(__uint_as_float(a) * 512.0f);   // < 2^-6
  return sgn | (((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3));
}

// One w2 row per wave: the row's largest magnitude, its FP16 scale
// RN16(max / 448), and every element's code of w / scale (zero codes when the
// scale is 0).
__global__ __launch_bounds__(256) void quantize_w2_fp8_kernel(const uint16_t* w2, uint8_t* q,
                                                              uint16_t* scales, int V, int R) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= V) return;
  const uint16_t* w = w2 + (size_t)row * R;
  float amax = 0.0f;
  for (int j = lane; j < R; j += 64) amax = fmaxf(amax, fabsf(__uint_as_float((uint32_t)w[j] << 16)));
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) amax = fmaxf(amax, __shfl_xor(amax, sh));
  const _Float16 sh16 = (_Float16)(amax / 448.0f);
  const float scale = (float)sh16;
  for (int j = lane; j < R; j += 64)
    q[(size_t)row * R + j] =
        scale == 0.0f ? (uint8_t)0 : (uint8_t)e4m3_encode(__uint_as_float((uint32_t)w[j] << 16) / scale);
  if (lane == 0) scales[row] = __builtin_bit_cast(uint16_t, sh16);
}

__global__ void debug_e4m3_encode_kernel(const float* x, uint8_t* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint8_t)e4m3_encode(x[i]);
}

// 8 codes per thread through the step kernel's own decode (decode8).
__global__ void debug_e4m3_decode_kernel(const uint2* codes, bf16x8_t* out, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n8) out[i] = decode8(codes[i].x, codes[i].y);
}

// A row's token over G vocabulary shards: the largest packed winner (the
// packing orders as the total order, global ids included) decoded.
__global__ __launch_bounds__(256) void pick_kernel(const unsigned long long* packets, int G, int rows,
                                                   int64_t* tokens, int64_t stride,
                                                   unsigned long long* winner) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  unsigned long long w = 0ull;
  for (int g = 0; g < G; ++g) {
    const unsigned long long c = packets[(size_t)g * rows + r];
    w = c > w ? c : w;
  }
  tokens[(int64_t)r * stride] = slot_token(w);
  if (winner) winner[r] = w;
}

// The packed winners' token ids (the low word holds ~id).
__global__ __launch_bounds__(256) void finalize_kernel(const unsigned long long* winners, int64_t n,
                                                       int64_t* tokens) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) tokens[i] = slot_token(winners[i]);
}

// ---------------------------------------------------------------- no-alloc variant
//
// For callers that cannot allocate device memory: the workspace is this
// library's own file-scope array, one per GPU the library runs on (held until
// the process ends), sized for the most rows any rank takes. Host code never
// passes the array's name to a kernel or a copy: it takes the array's device
// address from hipGetSymbolAddress once per device and uses that.
constexpr int32_t NOALLOC_MAX_ROWS = ROWS_CAP;
constexpr size_t NOALLOC_BYTES = (size_t)WS_SLOTS + (size_t)NOALLOC_MAX_ROWS * 8 * 3 * SG;
static __device__ __align__(256) unsigned char scratch[NOALLOC_BYTES];

__global__ __launch_bounds__(256) void zero_kernel(u32x4_t* p, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = (u32x4_t){0u, 0u, 0u, 0u};
}

struct ScratchState {
  void* ptr = nullptr;          // the device address of `scratch` on this device
  bool tables = false;          // noise bound tables copied in
  bool stamped = false;         // a transform table is in, for (mult_bits, cap_bits)
  uint32_t mult_bits = 0, cap_bits = 0;
};
constexpr int NOALLOC_DEVICES = 64;
ScratchState g_scratch[NOALLOC_DEVICES];
std::mutex g_scratch_mutex;

// The scratch of the current device, prepared for a call of this shape: set
// up once per device (its address, the noise bound tables), the transform
// table copied in when the call's (mult, softcap) differ from the one in it,
// and the ticket and the slots of `rows` rows cleared by a fill kernel.
int scratch_for(const markov_shape_t* sh, hipStream_t st, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MARKOV_ERR_HIP;
  if (dev < 0 || dev >= NOALLOC_DEVICES) return MARKOV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  ScratchState& S = g_scratch[dev];
  if (!S.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MARKOV_ERR_HIP;
    S.ptr = p;
  }
  unsigned char* ws = (unsigned char*)S.ptr;
  if (!S.tables) {
    build_table();
    if (hipMemcpyAsync(ws, g_table, GT_BYTES, hipMemcpyHostToDevice, st) != hipSuccess ||
        hipMemcpyAsync(ws + GT_BYTES, g_ctable, GTC_BYTES, hipMemcpyHostToDevice, st) != hipSuccess)
      return MARKOV_ERR_HIP;
    S.tables = true;
  }
  if (sh->softcap > 0.0f) {
    uint32_t mb, cb;
    memcpy(&mb, &sh->mult, 4);
    memcpy(&cb, &sh->softcap, 4);
    if (!S.stamped || S.mult_bits != mb || S.cap_bits != cb) {
      const TransformTable* t = transform_table(sh->mult, sh->softcap);
      if (hipMemcpyAsync(ws + WS_TT, t->data, TT_HEAD + TT_BYTES, hipMemcpyHostToDevice, st) !=
          hipSuccess)
        return MARKOV_ERR_HIP;
      S.stamped = true;
      S.mult_bits = mb;
      S.cap_bits = cb;
    }
  }
  const int64_t n16 = (int64_t)(ws_bytes(sh->rows) - WS_TICKET) / 16;
  zero_kernel<<<dim3((unsigned)((n16 + 255) / 256)), 256, 0, st>>>((u32x4_t*)(ws + WS_TICKET), n16);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  *out = S.ptr;
  return MARKOV_OK;
}

}  // namespace

extern "C" {

int32_t markov_max_rows(int32_t rank) { return max_rows_of(rank); }

size_t markov_workspace_bytes(const markov_shape_t* shape, int32_t k) {
  if (check_shape(shape, k)) return 0;
  return ws_bytes(shape->rows);
}

int markov_workspace_init(void* workspace, size_t bytes, const markov_shape_t* shape,
                          markov_stream_t stream) {
  if (!workspace) return MARKOV_ERR_NULL;
  if (!aligned16(workspace)) return MARKOV_ERR_ALIGN;
  if (bytes < ws_bytes(1)) return MARKOV_ERR_WORKSPACE;
  build_table();
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(ws, g_table, GT_BYTES, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipMemcpyAsync(ws + GT_BYTES, g_ctable, GTC_BYTES, hipMemcpyHostToDevice, st) != hipSuccess)
    return MARKOV_ERR_HIP;
  if (shape && shape->softcap > 0.0f) {
    const TransformTable* t = transform_table(shape->mult, shape->softcap);
    if (hipMemcpyAsync(ws + WS_TT, t->data, TT_HEAD + TT_BYTES, hipMemcpyHostToDevice, st) != hipSuccess)
      return MARKOV_ERR_HIP;
  } else if (hipMemsetAsync(ws + WS_TT, 0, TT_HEAD, st) != hipSuccess) {   // no stamp
    return MARKOV_ERR_HIP;
  }
  if (hipMemsetAsync(ws + WS_TICKET, 0, bytes - WS_TICKET, st) != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

const char* markov_why_not(const markov_shape_t* shape, int32_t k) {
  if (!shape) return "no shape";
  if (shape->rows < 1) return "no requests";
  if (k < 1) return "no draft steps";
  if (shape->vocab < 1 || (shape->vocab & 7)) return "vocabulary not a positive multiple of 8";
  if (shape->vocab > MARKOV_MAX_VOCAB) return "vocabulary above MARKOV_MAX_VOCAB";
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

int markov_sample_sequential_noalloc(const void* base_logits, const void* w1, const void* w2,
                                     const int64_t* prev, const int64_t* seeds,
                                     const int64_t* positions, int32_t k,
                                     const float* temperature, void* cache, int64_t* tokens,
                                     markov_stream_t stream, const markov_shape_t* shape) {
  int rc = check_shape(shape, k);
  if (rc) return rc;
  if (shape->rows > NOALLOC_MAX_ROWS || ws_bytes(shape->rows) > NOALLOC_BYTES)
    return MARKOV_ERR_WORKSPACE;
  if (!base_logits || !w1 || !w2 || !prev || !seeds || !positions || !temperature || !cache ||
      !tokens)
    return MARKOV_ERR_NULL;
  if (!aligned16(base_logits) || !aligned16(w1) || !aligned16(w2) || !aligned16(cache))
    return MARKOV_ERR_ALIGN;
  void* ws = nullptr;
  rc = scratch_for(shape, (hipStream_t)stream, &ws);
  if (rc) return rc;
  return sample_common(MODE_SAMPLE, base_logits, w1, w2, prev, seeds, positions, k, 0, k,
                       temperature, cache, tokens, stream, shape, ws, NOALLOC_BYTES);
}

int32_t markov_noalloc_max_rows(void) { return NOALLOC_MAX_ROWS; }

int markov_greedy_sequential(const void* base_logits, const void* w1, const void* w2,
                             const int64_t* prev, int32_t k, void* cache, int64_t* tokens,
                             uint64_t* winners, markov_stream_t stream,
                             const markov_shape_t* shape, void* workspace,
                             size_t workspace_bytes) {
  return greedy_common(base_logits, w1, w2, prev, k, 0, k, cache, tokens,
                       (unsigned long long*)winners, stream, shape, workspace, workspace_bytes);
}

int markov_greedy_step(const void* base_logits, const void* w1, const void* w2,
                       const int64_t* prev, int32_t k, int32_t step, void* cache, int64_t* tokens,
                       uint64_t* winners, markov_stream_t stream, const markov_shape_t* shape,
                       void* workspace, size_t workspace_bytes) {
  return greedy_common(base_logits, w1, w2, prev, k, step, step + 1, cache, tokens,
                       (unsigned long long*)winners, stream, shape, workspace, workspace_bytes);
}

int markov_quantize_w2_fp8(const void* w2, uint8_t* w2q, uint16_t* w2_scales, int32_t vocab,
                           int32_t rank, markov_stream_t stream) {
  if (vocab < 1 || !pow2_rank(rank)) return vocab < 1 ? MARKOV_ERR_SHAPE : MARKOV_ERR_RANK;
  if (vocab > MARKOV_MAX_VOCAB) return MARKOV_ERR_VOCAB;
  if (!w2 || !w2q || !w2_scales) return MARKOV_ERR_NULL;
  const unsigned blocks = (unsigned)((vocab + 3) / 4);
  quantize_w2_fp8_kernel<<<dim3(blocks), 256, 0, (hipStream_t)stream>>>(
      (const uint16_t*)w2, w2q, w2_scales, vocab, rank);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

int markov_sample_sequential_fp8(const void* base_logits, const void* w1, const uint8_t* w2q,
                                 const uint16_t* w2_scales, const int64_t* prev,
                                 const int64_t* seeds, const int64_t* positions, int32_t k,
                                 const float* temperature, void* cache, int64_t* tokens,
                                 markov_stream_t stream, const markov_shape_t* shape,
                                 void* workspace, size_t workspace_bytes) {
  if (!w2q || !w2_scales) return MARKOV_ERR_NULL;
  return sample_common(MODE_SAMPLE, base_logits, w1, nullptr, prev, seeds, positions, k, 0, k,
                       temperature, cache, tokens, stream, shape, workspace, workspace_bytes, w2q,
                       w2_scales);
}

int markov_greedy_sequential_fp8(const void* base_logits, const void* w1, const uint8_t* w2q,
                                 const uint16_t* w2_scales, const int64_t* prev, int32_t k,
                                 void* cache, int64_t* tokens, uint64_t* winners,
                                 markov_stream_t stream, const markov_shape_t* shape,
                                 void* workspace, size_t workspace_bytes) {
  if (!w2q || !w2_scales) return MARKOV_ERR_NULL;
  return greedy_common(base_logits, w1, nullptr, prev, k, 0, k, cache, tokens,
                       (unsigned long long*)winners, stream, shape, workspace, workspace_bytes,
                       w2q, w2_scales);
}

int markov_sample_step_fp8(const void* base_logits, const void* w1, const uint8_t* w2q,
                           const uint16_t* w2_scales, const int64_t* prev, const int64_t* seeds,
                           const int64_t* positions, int32_t k, int32_t step,
                           const float* temperature, void* cache, int64_t* tokens,
                           markov_stream_t stream, const markov_shape_t* shape, void* workspace,
                           size_t workspace_bytes) {
  if (!w2q || !w2_scales) return MARKOV_ERR_NULL;
  return sample_common(MODE_SAMPLE, base_logits, w1, nullptr, prev, seeds, positions, k, step,
                       step + 1, temperature, cache, tokens, stream, shape, workspace,
                       workspace_bytes, w2q, w2_scales);
}

int markov_greedy_step_fp8(const void* base_logits, const void* w1, const uint8_t* w2q,
                           const uint16_t* w2_scales, const int64_t* prev, int32_t k, int32_t step,
                           void* cache, int64_t* tokens, uint64_t* winners, markov_stream_t stream,
                           const markov_shape_t* shape, void* workspace, size_t workspace_bytes) {
  if (!w2q || !w2_scales) return MARKOV_ERR_NULL;
  return greedy_common(base_logits, w1, nullptr, prev, k, step, step + 1, cache, tokens,
                       (unsigned long long*)winners, stream, shape, workspace, workspace_bytes,
                       w2q, w2_scales);
}

int markov_shard_step(const void* base_logits, const void* w1, const void* w2, const int64_t* feed,
                      int64_t feed_stride, const int64_t* seeds, const int64_t* positions,
                      int32_t k, int32_t step, const float* temperature, void* cache,
                      uint64_t* packets, int32_t vocab_offset, int32_t vocab_total,
                      markov_stream_t stream, const markov_shape_t* shape, void* workspace,
                      size_t workspace_bytes) {
  int rc = check_shape(shape, k);
  if (rc) return rc;
  if (step < 0 || step >= k || feed_stride < 1 || vocab_offset < 0 || vocab_total < 1 ||
      (int64_t)vocab_offset + shape->vocab > (int64_t)vocab_total)
    return MARKOV_ERR_SHAPE;
  if (vocab_total > MARKOV_MAX_VOCAB) return MARKOV_ERR_VOCAB;
  if (!base_logits || !w1 || !w2 || !feed || !seeds || !positions || !temperature || !cache ||
      !packets || !workspace)
    return MARKOV_ERR_NULL;
  if (!aligned16(base_logits) || !aligned16(w1) || !aligned16(w2) || !aligned16(cache) ||
      !aligned16(workspace))
    return MARKOV_ERR_ALIGN;
  if (workspace_bytes < ws_bytes(shape->rows)) return MARKOV_ERR_WORKSPACE;
  Call c;
  c.mode = MODE_SAMPLE;
  c.var = V_SAMPLE;
  c.base = base_logits;
  c.w1 = w1;
  c.w2 = w2;
  c.prev = feed;
  c.feed_stride = feed_stride;
  c.seeds = seeds;
  c.positions = positions;
  c.temperature = temperature;
  c.cache = cache;
  c.packets = (unsigned long long*)packets;
  c.id_offset = vocab_offset;
  c.vocab_total = vocab_total;
  c.k = k;
  c.s_begin = step;
  c.s_end = step + 1;
  return launch_steps(c, stream, shape, workspace);
}

int markov_pick(const uint64_t* packets, int32_t shards, int32_t rows, int64_t* tokens,
                int64_t stride, uint64_t* winner, markov_stream_t stream) {
  if (shards < 1 || rows < 1 || stride < 1) return MARKOV_ERR_SHAPE;
  if (!packets || !tokens) return MARKOV_ERR_NULL;
  pick_kernel<<<dim3((unsigned)((rows + 255) / 256)), 256, 0, (hipStream_t)stream>>>(
      (const unsigned long long*)packets, shards, rows, tokens, stride,
      (unsigned long long*)winner);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

int markov_debug_e4m3_encode(const float* x, uint8_t* out, int64_t n, markov_stream_t stream) {
  if (n < 0) return MARKOV_ERR_SHAPE;
  if (n == 0) return MARKOV_OK;
  if (!x || !out) return MARKOV_ERR_NULL;
  debug_e4m3_encode_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, (hipStream_t)stream>>>(x, out, n);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

int markov_debug_e4m3_decode(const uint8_t* codes, void* out, int64_t n, markov_stream_t stream) {
  if (n < 0 || (n & 7)) return MARKOV_ERR_SHAPE;
  if (n == 0) return MARKOV_OK;
  if (!codes || !out) return MARKOV_ERR_NULL;
  if (((uintptr_t)codes & 7u) || !aligned16(out)) return MARKOV_ERR_ALIGN;
  const int64_t n8 = n / 8;
  debug_e4m3_decode_kernel<<<dim3((unsigned)((n8 + 255) / 256)), 256, 0, (hipStream_t)stream>>>(
      (const uint2*)codes, (bf16x8_t*)out, n8);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

int markov_debug_bias_fp8(const void* w1, const uint8_t* w2q, const uint16_t* w2_scales,
                          const int64_t* tok, void* bias, const markov_shape_t* shape,
                          markov_stream_t stream) {
  int rc = check_shape(shape, 1);
  if (rc) return rc;
  if (!w1 || !w2q || !w2_scales || !tok || !bias) return MARKOV_ERR_NULL;
  if (!aligned16(w1) || !aligned16(w2q) || !aligned16(w2_scales) || !aligned16(bias))
    return MARKOV_ERR_ALIGN;
  Call c;
  c.mode = MODE_BIAS;
  c.var = V_W8;
  c.w1 = w1;
  c.w2q = w2q;
  c.w2s = w2_scales;
  c.prev = tok;
  c.bias_out = bias;
  return launch_steps(c, stream, shape, nullptr);
}

int markov_greedy_finalize(const uint64_t* winners, int64_t n, int64_t* tokens,
                           markov_stream_t stream) {
  if (n < 0) return MARKOV_ERR_SHAPE;
  if (n == 0) return MARKOV_OK;
  if (!winners || !tokens) return MARKOV_ERR_NULL;
  finalize_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, (hipStream_t)stream>>>(
      (const unsigned long long*)winners, n, tokens);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
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
    case MARKOV_ERR_ALIGN: return "a bf16 array or the workspace is not 16-byte aligned";
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
  Call c;
  c.mode = MODE_BIAS;
  c.w1 = w1;
  c.w2 = w2;
  c.prev = tok;
  c.bias_out = bias;
  return launch_steps(c, stream, shape, nullptr);
}

int markov_debug_gumbel(const float* logits, const uint32_t* ids, int64_t n, float temperature,
                        int64_t seed, int32_t step, int64_t position, const void* workspace,
                        float* key_exact_out, float* key_upper_out, markov_stream_t stream) {
  if (!logits || !ids || !workspace || !key_exact_out || !key_upper_out) return MARKOV_ERR_NULL;
  if (n < 0) return MARKOV_ERR_SHAPE;
  if (n == 0) return MARKOV_OK;
  const int tb = 256;
  const int64_t blocks = (n + tb - 1) / tb;
  debug_gumbel_kernel<<<dim3((unsigned)blocks), tb, 0, (hipStream_t)stream>>>(
      logits, ids, n, temperature, seed, step, position, (const float2*)workspace, key_exact_out,
      key_upper_out);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

int32_t markov_debug_noise_table(float* out, int32_t n) {
  if (!out) return MARKOV_ERR_NULL;
  build_table();
  const int32_t c = n < GT_N ? n : GT_N;
  for (int32_t i = 0; i < c; ++i) {
    out[3 * i] = g_table[i].x;
    out[3 * i + 1] = g_table[i].y;
    out[3 * i + 2] = g_ctable[i];
  }
  return c;
}

int32_t markov_debug_transform_table(float mult, float softcap, uint16_t* out, int32_t n) {
  if (!out) return MARKOV_ERR_NULL;
  if (!(softcap > 0.0f) || n < 0) return MARKOV_ERR_SHAPE;
  const TransformTable* t = transform_table(mult, softcap);
  const int32_t c = n < (int32_t)(TT_BYTES / 2) ? n : (int32_t)(TT_BYTES / 2);
  memcpy(out, (const unsigned char*)t->data + TT_HEAD, (size_t)c * 2);
  return c;
}

int markov_debug_copy(const void* src, void* dst, int64_t bytes, markov_stream_t stream) {
  if (!src || !dst) return MARKOV_ERR_NULL;
  if (bytes < 0 || (bytes & 15)) return MARKOV_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return MARKOV_ERR_ALIGN;
  if (bytes == 0) return MARKOV_OK;
  const int64_t n16 = bytes / 16;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
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
