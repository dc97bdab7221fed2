// MI355X (gfx950) verification of a drafted block (TensorRT Edge-LLM "DSpark
// kernels" page: `dsparkGreedyAccept`, `dsparkProbabilisticAccept`).
//
// Both verifiers are one launch each, spread over workgroups that each read
// one slice of a vocabulary row (the rows are large and few):
//   * greedy: a workgroup per (batch row, verify position, vocabulary chunk)
//     reduces its slice of the bf16 target logits to the first NaN, else the
//     lowest id of the largest value, and publishes it as one packed 64-bit
//     atomicMax (an order-preserving key, then the complement of the id);
//     positions past the row's proposal length are skipped;
//   * probabilistic: a workgroup per (batch row, vocabulary chunk) finds the
//     first rejected proposal (the speculative-sampling test u q < p, exact
//     in binary64), then the binary64 sum of its slice of the residual
//     max(0, p - q) (or of p_L when every proposal passed);
// and in both the workgroup that arrives last at its row's ticket (an
// agent-scope acquire-release fetch-add: every other workgroup's results
// are visible to it) finishes the row: the greedy acceptance scan, or the
// inverse-CDF search over the chunk sums and then inside the chunk that holds
// the threshold. It re-zeroes what it used, so the workspace stays zeroed.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "markov.h"

namespace {

constexpr int VT = 256;             // threads per verifier workgroup
constexpr int VCHUNKS = 8;          // vocabulary chunks per row

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

// grid: (chunks, P + 1, B). Workspace: slots [B][P+1] u64, tickets [B] u32.
__global__ __launch_bounds__(VT) void greedy_accept_kernel(
    const uint16_t* logits, const int64_t* draft, const int32_t* lengths, int64_t* accepted,
    int32_t* accept_len, unsigned long long* slots, unsigned int* tickets, int P, int V,
    int draft_stride, int chunks) {
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int L = lengths[b];
  L = L < 0 ? 0 : L > P ? P : L;
  __shared__ float sv[VT / 64];
  __shared__ int si[VT / 64];
  __shared__ int last;
  if (j <= L) {
    // this chunk of the row: 8 bf16 per 16-byte load, ids ascending per thread
    const int per = ((V / 8 + chunks - 1) / chunks);
    const int q0 = c * per, q1 = min(V / 8, q0 + per);
    const uint16_t* row = logits + ((size_t)b * (P + 1) + j) * V;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int q = q0 + tid; q < q1; q += VT) {
      const u32x4_t w = *(const u32x4_t*)(row + (size_t)q * 8);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float l = (e & 1) ? bf_hi(ws[e >> 1]) : bf_lo(ws[e >> 1]);
        if (before(l, q * 8 + e, bv, bi)) {
          bv = l;
          bi = q * 8 + e;
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
  // the row's ticket: every workgroup of row b counts, skipped positions too
  if (tid == 0) {
    const unsigned n = (unsigned)((P + 1) * chunks);
    last = __hip_atomic_fetch_add(tickets + b, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
           n - 1u;
  }
  __syncthreads();
  if (!last || tid != 0) return;
  int n = 0;
  int64_t bonus = 0;
  for (int jj = 0; jj <= L; ++jj) {
    const unsigned long long w = __hip_atomic_exchange(slots + (size_t)b * (P + 1) + jj, 0ull,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int64_t a = unpack_id(w);
    if (jj < L && draft[(size_t)b * draft_stride + jj] == a) {
      accepted[(size_t)b * (P + 1) + n++] = a;
      continue;
    }
    bonus = a;
    for (int k2 = jj + 1; k2 <= L; ++k2)   // slots the scan did not reach
      __hip_atomic_store(slots + (size_t)b * (P + 1) + k2, 0ull, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    break;
  }
  accepted[(size_t)b * (P + 1) + n++] = bonus;
  for (int i = n; i <= P; ++i) accepted[(size_t)b * (P + 1) + i] = -1;
  accept_len[b] = n;
  __hip_atomic_store(tickets + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- probabilistic

// The first rejected proposal of row b (L if none), as the oracle: accept
// iff u_j q_j(d) < p_j(d) in binary64 (both products exact); an id outside
// [0, V) has p = q = 0.
__device__ int first_reject(const float* target, const float* draftp, const int64_t* draft,
                            const float* uniforms, int b, int L, int P, int V, int draft_stride) {
  for (int j = 0; j < L; ++j) {
    const int64_t d = draft[(size_t)b * draft_stride + j];
    double p = 0.0, q = 0.0;
    if (d >= 0 && d < V) {
      p = (double)target[((size_t)b * (P + 1) + j) * V + d];
      q = (double)draftp[((size_t)b * P + j) * V + d];
    }
    if (!((double)uniforms[(size_t)b * (2 * P + 1) + j] * q < p)) return j;
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

// The smallest x in [x0, x1) whose running sum from `base` exceeds t: each
// thread sums a contiguous run, an exclusive scan of the runs finds the
// thread whose run holds the crossing, and it walks its run (the lowest
// crossing any thread finds wins). -1 if none.
__device__ int find_in(const float* prow, const float* qrow, bool resid, int x0, int x1, double base,
                       double t, double* red, int* found) {
  const int tid = threadIdx.x;
  const int per = (x1 - x0 + VT - 1) / VT;
  const int a = x0 + tid * per, e = min(x1, a + per);
  double s = 0.0;
  for (int x = a; x < e; ++x) s += weight(prow, qrow, resid, x);
  __syncthreads();
  red[tid] = s;
  if (tid == 0) *found = 0x7fffffff;
  __syncthreads();
  double pre = base;
  for (int i = 0; i < tid; ++i) pre += red[i];   // VT terms: small next to the row
  if (pre + s > t && pre <= t) {
    double cum = pre;
    for (int x = a; x < e; ++x) {
      cum += weight(prow, qrow, resid, x);
      if (cum > t) {
        atomicMin(found, x);
        break;
      }
    }
  }
  __syncthreads();
  const int f = *found;
  return f == 0x7fffffff ? -1 : f;
}

// grid: (chunks, B). Workspace: partial sums [B][chunks] f64, tickets [B].
__global__ __launch_bounds__(VT) void prob_accept_kernel(
    const float* target, const float* draftp, const int64_t* draft, const int32_t* lengths,
    const float* uniforms, int64_t* accepted, int32_t* accept_len, double* partial,
    unsigned int* tickets, int P, int V, int draft_stride, int chunks) {
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  __shared__ double red[VT];
  __shared__ int sj, last, found;
  int L = lengths[b];
  L = L < 0 ? 0 : L > P ? P : L;
  if (tid == 0) sj = first_reject(target, draftp, draft, uniforms, b, L, P, V, draft_stride);
  __syncthreads();
  const int j = sj;
  const bool resid = j < L;
  const float* prow = target + ((size_t)b * (P + 1) + j) * V;
  const float* qrow = resid ? draftp + ((size_t)b * P + j) * V : nullptr;
  const int per = (V + chunks - 1) / chunks;
  const int x0 = c * per, x1 = min(V, x0 + per);
  double s = 0.0;
  for (int x = x0 + tid; x < x1; x += VT) s += weight(prow, qrow, resid, x);
  s = block_sum(s, red);
  if (tid == 0) {
    __hip_atomic_store(partial + (size_t)b * chunks + c, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = __hip_atomic_fetch_add(tickets + b, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
           (unsigned)chunks - 1u;
  }
  __syncthreads();
  if (!last) return;
  // the row's finisher: S over the chunks in order, the threshold u S, the
  // chunk that holds it, then the element
  double S = 0.0;
  for (int i = 0; i < chunks; ++i)
    S += __hip_atomic_load(partial + (size_t)b * chunks + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool rs = resid;
  const float u = uniforms[(size_t)b * (2 * P + 1) + (resid ? P + j : 2 * P)];
  int x = -1;
  if (!(S > 0.0) && rs) {       // no residual mass: sample p itself
    rs = false;
    double s2 = 0.0;
    for (int y = tid; y < V; y += VT) s2 += (double)prow[y];
    S = block_sum(s2, red);
  }
  if (S > 0.0) {
    const double t = (double)u * S;
    double base = 0.0;
    int cc = 0;
    for (; cc < chunks; ++cc) {   // the chunk sums of the first pass, or p's
      double cs;
      if (rs == resid) {
        cs = __hip_atomic_load(partial + (size_t)b * chunks + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        const int a0 = cc * per, a1 = min(V, a0 + per);
        double s3 = 0.0;
        for (int y = a0 + tid; y < a1; y += VT) s3 += (double)prow[y];
        cs = block_sum(s3, red);
      }
      if (base + cs > t) break;
      base += cs;
    }
    if (cc < chunks) x = find_in(prow, qrow, rs, cc * per, min(V, cc * per + per), base, t, red, &found);
    if (x < 0) {                  // rounding left the threshold at the end: the last weighted id
      const int a0 = cc < chunks ? cc * per : 0, a1 = cc < chunks ? min(V, a0 + per) : V;
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
    int n = 0;
    for (int i = 0; i < j; ++i) accepted[(size_t)b * (P + 1) + n++] = draft[(size_t)b * draft_stride + i];
    accepted[(size_t)b * (P + 1) + n++] = x;
    for (int i = n; i <= P; ++i) accepted[(size_t)b * (P + 1) + i] = -1;
    accept_len[b] = n;
    for (int i = 0; i < chunks; ++i)
      __hip_atomic_store(partial + (size_t)b * chunks + i, 0.0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(tickets + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t greedy_ws(int32_t B, int32_t P) { return ((size_t)B * (P + 1) * 8 + (size_t)B * 4 + 255) & ~(size_t)255; }
size_t prob_ws(int32_t B) { return ((size_t)B * VCHUNKS * 8 + (size_t)B * 4 + 255) & ~(size_t)255; }

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
  if (batch < 1 || proposal_len < 0 || vocab < 8 || (vocab & 7) || draft_stride < proposal_len)
    return MARKOV_ERR_SHAPE;
  if (!target_logits || (proposal_len > 0 && !draft) || !proposal_lengths || !accepted ||
      !accept_len || !workspace)
    return MARKOV_ERR_NULL;
  if (!aligned16(target_logits) || !aligned16(workspace)) return MARKOV_ERR_ALIGN;
  if (workspace_bytes < markov_verify_workspace_bytes(batch, proposal_len)) return MARKOV_ERR_WORKSPACE;
  unsigned long long* slots = (unsigned long long*)workspace;
  unsigned int* tickets = (unsigned int*)(slots + (size_t)batch * (proposal_len + 1));
  const int chunks = vocab / 8 >= VCHUNKS * VT ? VCHUNKS : 1;
  dim3 grid((unsigned)chunks, (unsigned)(proposal_len + 1), (unsigned)batch);
  greedy_accept_kernel<<<grid, VT, 0, (hipStream_t)stream>>>(
      (const uint16_t*)target_logits, draft, proposal_lengths, accepted, accept_len, slots, tickets,
      proposal_len, vocab, draft_stride, chunks);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

int markov_prob_accept(const float* target_probs, const float* draft_probs, const int64_t* draft,
                       int32_t draft_stride, const int32_t* proposal_lengths, const float* uniforms,
                       int64_t* accepted, int32_t* accept_len, int32_t batch, int32_t proposal_len,
                       int32_t vocab, void* workspace, size_t workspace_bytes,
                       markov_stream_t stream) {
  if (batch < 1 || proposal_len < 0 || vocab < 1 || draft_stride < proposal_len)
    return MARKOV_ERR_SHAPE;
  if (!target_probs || !proposal_lengths || !uniforms || !accepted || !accept_len || !workspace ||
      (proposal_len > 0 && (!draft_probs || !draft)))
    return MARKOV_ERR_NULL;
  if (!aligned16(workspace)) return MARKOV_ERR_ALIGN;
  if (workspace_bytes < markov_verify_workspace_bytes(batch, proposal_len)) return MARKOV_ERR_WORKSPACE;
  double* partial = (double*)workspace;
  unsigned int* tickets = (unsigned int*)(partial + (size_t)batch * VCHUNKS);
  const int chunks = VCHUNKS;
  dim3 grid((unsigned)chunks, (unsigned)batch);
  prob_accept_kernel<<<grid, VT, 0, (hipStream_t)stream>>>(
      target_probs, draft_probs, draft, proposal_lengths, uniforms, accepted, accept_len, partial,
      tickets, proposal_len, vocab, draft_stride, chunks);
  if (hipGetLastError() != hipSuccess) return MARKOV_ERR_HIP;
  return MARKOV_OK;
}

}  // extern "C"
