// MI355X (gfx950) verification of a drafted block (TensorRT Edge-LLM "DSpark
// kernels" page: `dsparkGreedyAccept`, `dsparkProbabilisticAccept`).
//
// Each verifier is two launches: a wide pass over workgroups that each read
// one slice of a vocabulary row (the rows are large and few), then one
// workgroup per batch row that finishes it. The kernel boundary orders the
// two, so no workgroup needs a device-scope fence (an agent-scope release in
// every workgroup of the wide pass -- an L2 write-back each -- cost more than
// the pass itself).
//   * greedy: a workgroup per (batch row, verify position, vocabulary chunk)
//     reduces its slice of the bf16 target logits to the first NaN, else the
//     lowest id of the largest value, and publishes it as one packed 64-bit
//     atomicMax (an order-preserving key, then the complement of the id) into
//     the position's slot; positions past the row's proposal length are
//     skipped. The finisher scans the slots (the acceptance test) and zeroes
//     them.
//   * probabilistic: a workgroup per (batch row, vocabulary chunk) finds the
//     first rejected proposal (the speculative-sampling test u q < p, exact
//     in binary64) and stores the binary64 sum of its slice of the residual
//     max(0, p - q) (or of p_L when every proposal passed); the row's first
//     chunk also records that proposal and its uniform. The finisher adds
//     the chunk sums in order, finds the chunk that holds the threshold u S,
//     then the element, and zeroes the sums and the record.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "markov.h"

namespace {

constexpr int VT = 256;             // threads per verifier workgroup
constexpr int VCHUNKS = 8;          // vocabulary chunks per row (greedy)
constexpr int PCHUNKS = 32;         // the most vocabulary chunks per row (probabilistic)
constexpr int RPMAX = 32;           // the longest per-thread run the finisher keeps in LDS

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// (v1, i1) before (v2, i2): a NaN first (lower id among NaNs), else the
// larger value, equal values (-0 == +0) to the lower id.
__device__ __forceinline__ bool before(float v1, int64_t i1, float v2, int64_t i2) {
  const bool n1 = __builtin_isnan(v1), n2 = __builtin_isnan(v2);
  return (v1 > v2) || (v1 == v2 && i1 < i2) || (n1 && (!n2 || i1 < i2));
}

// The order-preserving image of (v, id): every NaN at the top, -0 as +0,
// then the complement of the id (equal values favour the lower id); 0 is
// below every real element.
__device__ __forceinline__ unsigned long long pack(float v, int64_t id) {
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

__device__ __forceinline__ int64_t unpack_id(unsigned long long w) {
  return (int64_t)(uint32_t)(~(uint32_t)w);
}

// ---------------------------------------------------------------- greedy

// grid: (chunks, P + 1, B). Workspace: slots [B][P+1] u64 (zero between calls).
__global__ __launch_bounds__(VT) void greedy_accept_kernel(const uint16_t* logits,
                                                           const int32_t* lengths,
                                                           unsigned long long* slots, int P, int V,
                                                           int chunks) {
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int L = lengths[b];
  L = L < 0 ? 0 : L > P ? P : L;
  __shared__ float sv[VT / 64];
  __shared__ int si[VT / 64];
  if (j <= L) {
    // this chunk of the row: 8 bf16 per 16-byte load, ids ascending per thread
    const int per = ((V / 8 + chunks - 1) / chunks);
    const int q0 = c * per, q1 = min(V / 8, q0 + per);
    const uint16_t* row = logits + ((size_t)b * (P + 1) + j) * V;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    // GU loads in flight per thread before any is used. A thread meets its
    // elements in rising id, so one is taken over the kept one iff the kept
    // one is not NaN and it is NaN or larger (a tie keeps the earlier id);
    // a thread whose elements are all -inf takes none, and then its first
    // (the lowest id among equal values) below.
    constexpr int GU = 4;
    for (int q = q0 + tid; q < q1; q += GU * VT) {
      u32x4_t w[GU];
#pragma unroll
      for (int u = 0; u < GU; ++u)
        w[u] = q + u * VT < q1 ? *(const u32x4_t*)(row + (size_t)(q + u * VT) * 8) : (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        if (q + u * VT >= q1) break;
        const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
        const int id0 = (q + u * VT) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float l = (e & 1) ? bf_hi(ws[e >> 1]) : bf_lo(ws[e >> 1]);
          const bool take = !__builtin_isnan(bv) & (__builtin_isnan(l) | (l > bv));
          bv = take ? l : bv;
          bi = take ? id0 + e : bi;
        }
      }
    }
    if (bi == 0x7fffffff && q0 + tid < q1) bi = (q0 + tid) * 8;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const float ov = __shfl_xor(bv, sh);
      const int oi = __shfl_xor(bi, sh);
      if (before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      sv[wave] = bv;
      si[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w2 = 1; w2 < VT / 64; ++w2)
        if (before(sv[w2], si[w2], bv, bi)) {
          bv = sv[w2];
          bi = si[w2];
        }
      if (bi != 0x7fffffff)
        __hip_atomic_fetch_max(slots + (size_t)b * (P + 1) + j, pack(bv, bi), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// One thread per batch row: the acceptance scan over the row's slots.
__global__ __launch_bounds__(64) void greedy_finish_kernel(const int64_t* draft, const int32_t* lengths,
                                                           int64_t* accepted, int32_t* accept_len,
                                                           unsigned long long* slots, int B, int P,
                                                           int draft_stride) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int L = lengths[b];
  L = L < 0 ? 0 : L > P ? P : L;
  unsigned long long* sl = slots + (size_t)b * (P + 1);
  int n = 0;
  int64_t bonus = 0;
  int jj = 0;
  for (; jj <= L; ++jj) {
    const int64_t a = unpack_id(sl[jj]);
    if (jj < L && draft[(size_t)b * draft_stride + jj] == a) {
      accepted[(size_t)b * (P + 1) + n++] = a;
      continue;
    }
    bonus = a;
    break;
  }
  accepted[(size_t)b * (P + 1) + n++] = bonus;
  for (int i = n; i <= P; ++i) accepted[(size_t)b * (P + 1) + i] = -1;
  accept_len[b] = n;
  for (int i = 0; i <= L; ++i) sl[i] = 0ull;   // the slots this call filled
}

// ---------------------------------------------------------------- probabilistic

// The first rejected proposal of row b (L if none), as the oracle: accept
// iff u_j q_j(d) < p_j(d) in binary64 (both products exact); an id outside
// [0, V) has p = q = 0.
// Called by a whole wave: lane j tests proposal j (64 at a time), so the
// loads of every proposal are in flight together; the proposals and their
// uniforms do not wait for L (only their test does).
__device__ int first_reject(const float* target, const float* draftp, const int64_t* draft,
                            const float* uniforms, int b, int L, int P, int V, int draft_stride) {
  const int lane = threadIdx.x & 63;
  for (int j0 = 0; j0 < P; j0 += 64) {
    const int j = j0 + lane;
    int64_t d = -1;
    float uj = 0.0f;
    if (j < P) {
      d = draft[(size_t)b * draft_stride + j];
      uj = uniforms[(size_t)b * (2 * P + 1) + j];
    }
    if (j0 >= L) break;
    bool rej = false;
    if (j < L) {
      double p = 0.0, q = 0.0;
      if (d >= 0 && d < V) {
        p = (double)target[((size_t)b * (P + 1) + j) * V + d];
        q = (double)draftp[((size_t)b * P + j) * V + d];
      }
      rej = !((double)uj * q < p);
    }
    const unsigned long long m = __ballot(rej);
    if (m) return j0 + __builtin_ctzll(m);
  }
  return L;
}

// The sampling weight of x: the binary32 residual max(0, p - q) at a
// rejection, else p (resid = false).
__device__ __forceinline__ double weight(const float* prow, const float* qrow, bool resid, int x) {
  if (!resid) return (double)prow[x];
  const float r = prow[x] - qrow[x];
  return r > 0.0f ? (double)r : 0.0;
}

// This thread's binary64 sum of the weights of x = x0 + tid, x0 + tid +
// VT, ... < x1 in groups of four (16-byte loads, four groups in flight) when
// the row is 16-byte aligned and x0 a multiple of 4, else one by one.
__device__ double strided_sum(const float* prow, const float* qrow, bool resid, int x0, int x1) {
  const int tid = threadIdx.x;
  double s = 0.0;
  const bool vec = ((((uintptr_t)prow) | (uintptr_t)(resid ? qrow : prow)) & 15u) == 0 && (x0 & 3) == 0;
  if (vec) {
    const int g0 = x0 / 4, g1 = x1 / 4;
    for (int g = g0 + tid; g < g1; g += 4 * VT) {
      float4 pv[4], qv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = g + u * VT < g1;
        pv[u] = ok ? ((const float4*)prow)[g + u * VT] : make_float4(0.f, 0.f, 0.f, 0.f);
        qv[u] = ok && resid ? ((const float4*)qrow)[g + u * VT] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float a[4] = {pv[u].x, pv[u].y, pv[u].z, pv[u].w};
        const float b[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float r = resid ? a[e] - b[e] : a[e];
          s += resid ? (r > 0.0f ? (double)r : 0.0) : (double)r;
        }
      }
    }
    for (int x = 4 * g1 + tid; x < x1; x += VT) s += weight(prow, qrow, resid, x);
    return s;
  }
  for (int x = x0 + tid; x < x1; x += VT) s += weight(prow, qrow, resid, x);
  return s;
}

// Block-wide binary64 sum (every thread gets it).
__device__ double block_sum(double v, double* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) v += __shfl_xor(v, sh);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < VT / 64; ++w) t += red[w];
  return t;
}

// The binary64 sum, in index order, of the weights of [a, e): 16-byte loads
// four deep when the rows are 16-byte aligned and a is a multiple of 4. With
// STAGE, weight a + k also goes to st[k * VT] (as binary32: the weights are
// binary32 values, so the conversion back is exact).
template <bool STAGE>
__device__ double run_sum(const float* prow, const float* qrow, bool resid, int a, int e, float* st) {
  double s = 0.0;
  const bool vec = ((((uintptr_t)prow) | (uintptr_t)(resid ? qrow : prow)) & 15u) == 0 && (a & 3) == 0;
  int x = a;
  if (vec) {
    for (; x + 16 <= e; x += 16) {
      float4 pv[4], qv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pv[u] = ((const float4*)(prow + x))[u];
        qv[u] = resid ? ((const float4*)(qrow + x))[u] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float pa[4] = {pv[u].x, pv[u].y, pv[u].z, pv[u].w};
        const float qa[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float r = resid ? pa[k] - qa[k] : pa[k];
          const float w = resid ? (r > 0.0f ? r : 0.0f) : r;
          if (STAGE) st[(x - a + 4 * u + k) * VT] = w;
          s += (double)w;
        }
      }
    }
  }
  for (; x < e; ++x) {
    const double w = weight(prow, qrow, resid, x);
    if (STAGE) st[(x - a) * VT] = (float)w;
    s += w;
  }
  return s;
}

// The smallest x in [x0, x1) whose running sum from `base` exceeds t. Each
// thread sums a contiguous run (in index order); a block-wide exclusive scan
// of the run sums gives every run's starting sum B_i, so that the runs
// partition [base, B_VT) consistently (B is non-decreasing, the weights
// being non-negative); the thread whose [B_i, B_i+1) holds t walks its run
// from B_i, and where rounding leaves the walk short of t it takes the run's
// last weighted id. -1 if no run holds t.
// Runs of up to RPMAX weights stay in LDS between the sum and the walk.
__device__ int find_in(const float* prow, const float* qrow, bool resid, int x0, int x1, double base,
                       double t, double* red, int* found) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ double bnd[VT + 1];
  __shared__ float wst[RPMAX * VT];   // weight a + k of thread tid at [k * VT + tid]
  const int rp = (((x1 - x0 + VT - 1) / VT) + 3) & ~3;   // a multiple of 4
  const int a = min(x1, x0 + tid * rp), e = min(x1, a + rp);
  const bool staged = rp <= RPMAX;   // uniform
  const double s = staged ? run_sum<true>(prow, qrow, resid, a, e, wst + tid)
                          : run_sum<false>(prow, qrow, resid, a, e, nullptr);
  // exclusive scan: within the wave by shuffles, then the waves' totals
  double v = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  double ex = __shfl_up(v, 1);
  if (lane == 0) ex = 0.0;
  __syncthreads();
  if (lane == 63) red[wave] = v;
  if (tid == 0) *found = 0x7fffffff;
  __syncthreads();
  double before = base;
  for (int w = 0; w < wave; ++w) before += red[w];
  bnd[tid] = before + ex;
  if (tid == VT - 1) {
    double tot = base;
    for (int w = 0; w < VT / 64; ++w) tot += red[w];
    bnd[VT] = tot;
  }
  __syncthreads();
  const double b0 = bnd[tid], b1 = bnd[tid + 1];
  if (b0 <= t && t < b1) {
    // the walk over the run: its staged weights, else 16 loads at a time,
    // all in flight together
    double cum = b0;
    int hit = -1, last = -1;
    if (staged) {
      for (int x = a; x < e; ++x) {
        const double w = (double)wst[(x - a) * VT + tid];
        if (w > 0.0) last = x;
        cum += w;
        if (cum > t) {
          hit = x;
          break;
        }
      }
    } else {
      for (int x = a; x < e && hit < 0; x += 16) {
        double w[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) w[k] = x + k < e ? weight(prow, qrow, resid, x + k) : 0.0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          if (hit >= 0) break;
          if (w[k] > 0.0) last = x + k;
          cum += w[k];
          if (cum > t) hit = x + k;
        }
      }
    }
    atomicMin(found, hit >= 0 ? hit : last);
  }
  __syncthreads();
  const int f = *found;
  return f == 0x7fffffff || f < 0 ? -1 : f;
}

// A row's pick, recorded by its first chunk's workgroup: the first rejected
// proposal j (L if none), whether the row samples the residual (j < L), and
// the uniform of that sample.
struct RowPick {
  int32_t j, resid;
  float u;
  int32_t pad;
};

// grid: (chunks, B). Workspace: partial sums [B][PCHUNKS] f64 (row b's at
// b * chunks), then the picks [B] (all zero between calls).
__global__ __launch_bounds__(VT) void prob_accept_kernel(
    const float* target, const float* draftp, const int64_t* draft, const int32_t* lengths,
    const float* uniforms, double* partial, RowPick* pick, int P, int V, int draft_stride,
    int chunks) {
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  __shared__ double red[VT];
  __shared__ int sj;
  int L = lengths[b];
  L = L < 0 ? 0 : L > P ? P : L;
  if (tid < 64) {
    const int j0 = first_reject(target, draftp, draft, uniforms, b, L, P, V, draft_stride);
    if (tid == 0) sj = j0;
  }
  __syncthreads();
  const int j = sj;
  const bool resid = j < L;
  if (c == 0 && tid == 0)
    pick[b] = RowPick{j, resid ? 1 : 0, uniforms[(size_t)b * (2 * P + 1) + (resid ? P + j : 2 * P)], 0};
  const float* prow = target + ((size_t)b * (P + 1) + j) * V;
  const float* qrow = resid ? draftp + ((size_t)b * P + j) * V : nullptr;
  const int per = ((V + 4 * chunks - 1) / (4 * chunks)) * 4;   // a multiple of 4
  const int x0 = min(V, c * per), x1 = min(V, x0 + per);
  double s = block_sum(strided_sum(prow, qrow, resid, x0, x1), red);
  if (tid == 0) partial[(size_t)b * chunks + c] = s;
}

// One workgroup per batch row: S over the chunks in order, the threshold u S,
// the chunk that holds it, then the element; the chunk sums and the pick are
// re-zeroed. Everything it needs first (the pick and the sums) comes in one
// round trip.
__global__ __launch_bounds__(VT) void prob_finish_kernel(
    const float* target, const float* draftp, const int64_t* draft, int64_t* accepted,
    int32_t* accept_len, double* partial, RowPick* pick, int P, int V, int draft_stride, int chunks) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ double red[VT];
  __shared__ double csum[PCHUNKS];
  __shared__ RowPick sp;
  __shared__ int found;
  if (tid < chunks) csum[tid] = partial[(size_t)b * chunks + tid];   // the wide pass's chunk sums
  if (tid == 0) sp = pick[b];
  __syncthreads();
  const int j = sp.j;
  const bool resid = sp.resid != 0;
  const float u = sp.u;
  // the accepted drafts, then -1 past the sampled token (in flight during
  // the search)
  for (int i = tid; i <= P; i += VT) {
    if (i < j) accepted[(size_t)b * (P + 1) + i] = draft[(size_t)b * draft_stride + i];
    else if (i > j) accepted[(size_t)b * (P + 1) + i] = -1;
  }
  const float* prow = target + ((size_t)b * (P + 1) + j) * V;
  const float* qrow = resid ? draftp + ((size_t)b * P + j) * V : nullptr;
  const int per = ((V + 4 * chunks - 1) / (4 * chunks)) * 4;
  double S = 0.0;
  for (int i = 0; i < chunks; ++i) S += csum[i];
  bool rs = resid;
  int x = -1;
  if (!(S > 0.0) && rs) {       // no residual mass: sample p itself
    rs = false;
    S = block_sum(strided_sum(prow, nullptr, false, 0, V), red);
  }
  if (S > 0.0) {
    const double t = (double)u * S;
    double base = 0.0;
    int cc = 0;
    for (; cc < chunks; ++cc) {   // the chunk sums of the wide pass, or p's
      double cs;
      if (rs == resid) {
        cs = csum[cc];
      } else {
        const int a0 = min(V, cc * per), a1 = min(V, a0 + per);
        cs = block_sum(strided_sum(prow, nullptr, false, a0, a1), red);
      }
      if (base + cs > t) break;
      base += cs;
    }
    if (cc < chunks) x = find_in(prow, qrow, rs, min(V, cc * per), min(V, cc * per + per), base, t, red, &found);
    if (x < 0) {                  // rounding left the threshold at the end: the last weighted id
      const int a0 = cc < chunks ? min(V, cc * per) : 0, a1 = cc < chunks ? min(V, a0 + per) : V;
      if (tid == 0) {
        found = a0;
        for (int y = a1 - 1; y >= a0; --y)
          if (weight(prow, qrow, rs, y) > 0.0) {
            found = y;
            break;
          }
      }
      __syncthreads();
      x = found;
    }
  } else {
    x = 0;
  }
  if (tid == 0) {
    accepted[(size_t)b * (P + 1) + j] = x;
    accept_len[b] = j + 1;
    pick[b] = RowPick{0, 0, 0.0f, 0};
  }
  for (int i = tid; i < chunks; i += VT) partial[(size_t)b * chunks + i] = 0.0;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t greedy_ws(int32_t B, int32_t P) { return ((size_t)B * (P + 1) * 8 + 255) & ~(size_t)255; }
size_t prob_sums_bytes(int32_t B) { return ((size_t)B * PCHUNKS * 8 + 255) & ~(size_t)255; }
size_t prob_ws(int32_t B) { return prob_sums_bytes(B) + (((size_t)B * sizeof(RowPick) + 255) & ~(size_t)255); }

// chunks of a probabilistic row: about 4096 tokens each, 1 .. PCHUNKS
int prob_chunks(int32_t V) {
  const int c = V / 4096;
  return c < 1 ? 1 : c > PCHUNKS ? PCHUNKS : c;
}

}  // namespace

extern "C" {

size_t markov_verify_workspace_bytes(int32_t batch, int32_t proposal_len) {
  if (batch < 1 || proposal_len < 0) return 0;
  const size_t g = greedy_ws(batch, proposal_len), p = prob_ws(batch);
  return g > p ? g : p;
}

int markov_greedy_accept(const void* target_logits, const int64_t* draft, int32_t draft_stride,
                         const int32_t* proposal_lengths, int64_t* accepted, int32_t* accept_len,
                         int32_t batch, int32_t proposal_len, int32_t vocab, void* workspace,
                         size_t workspace_bytes, markov_stream_t stream) {
  if (vocab > MARKOV_MAX_VOCAB) return MARKOV_ERR_VOCAB;
  if (batch < 1 || proposal_len < 0 || vocab < 8 || (vocab & 7) || draft_stride < proposal_len)
    return MARKOV_ERR_SHAPE;
  if (!target_logits || (proposal_len > 0 && !draft) || !proposal_lengths || !accepted ||
      !accept_len || !workspace)
    return MARKOV_ERR_NULL;
  if (!aligned16(target_logits) || !aligned16(workspace)) return MARKOV_ERR_ALIGN;
  if (workspace_bytes < markov_verify_workspace_bytes(batch, proposal_len)) return MARKOV_ERR_WORKSPACE;
  unsigned long long* slots = (unsigned long long*)workspace;
  const int chunks = vocab / 8 >= VCHUNKS * VT ? VCHUNKS : 1;
  dim3 grid((unsigned)chunks, (unsigned)(proposal_len + 1), (unsigned)batch);
  greedy_accept_kernel<<<grid, VT, 0, (hipStream_t)stream>>>(
      (const uint16_t*)target_logits, proposal_lengths, slots, proposal_len, vocab, chunks);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  greedy_finish_kernel<<<dim3((unsigned)((batch + 63) / 64)), 64, 0, (hipStream_t)stream>>>(
      draft, proposal_lengths, accepted, accept_len, slots, batch, proposal_len, draft_stride);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

int markov_prob_accept(const float* target_probs, const float* draft_probs, const int64_t* draft,
                       int32_t draft_stride, const int32_t* proposal_lengths, const float* uniforms,
                       int64_t* accepted, int32_t* accept_len, int32_t batch, int32_t proposal_len,
                       int32_t vocab, void* workspace, size_t workspace_bytes,
                       markov_stream_t stream) {
  if (vocab > MARKOV_MAX_VOCAB) return MARKOV_ERR_VOCAB;
  if (batch < 1 || proposal_len < 0 || vocab < 1 || draft_stride < proposal_len)
    return MARKOV_ERR_SHAPE;
  if (!target_probs || !proposal_lengths || !uniforms || !accepted || !accept_len || !workspace ||
      (proposal_len > 0 && (!draft_probs || !draft)))
    return MARKOV_ERR_NULL;
  if (!aligned16(workspace)) return MARKOV_ERR_ALIGN;
  if (workspace_bytes < markov_verify_workspace_bytes(batch, proposal_len)) return MARKOV_ERR_WORKSPACE;
  double* partial = (double*)workspace;
  RowPick* pick = (RowPick*)((unsigned char*)workspace + prob_sums_bytes(batch));
  const int chunks = prob_chunks(vocab);
  prob_accept_kernel<<<dim3((unsigned)chunks, (unsigned)batch), VT, 0, (hipStream_t)stream>>>(
      target_probs, draft_probs, draft, proposal_lengths, uniforms, partial, pick, proposal_len,
      vocab, draft_stride, chunks);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  prob_finish_kernel<<<dim3((unsigned)batch), VT, 0, (hipStream_t)stream>>>(
      target_probs, draft_probs, draft, accepted, accept_len, partial, pick, proposal_len, vocab,
      draft_stride, chunks);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

}  // extern "C"
