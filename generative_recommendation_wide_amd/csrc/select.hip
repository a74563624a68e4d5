// Beam selection (xLLM generative-recommendation design doc, section 4.1.1: each beam
// expands top_k candidates, the next beam set is the best beam_width of the
// beam_width x top_k pool; section 4.3: stop unnecessary sorting early, filter invalid
// item paths early, reuse candidate containers; FlashRec announcement: with the fused
// semantic-ID trie illegal IDs are never candidates).
//
// Keys are compared as 64-bit composites (order-preserving float key, ~flat index), so one
// unsigned comparison orders by (key descending, flat index ascending) and every
// candidate is distinct: the selection is unique and deterministic whatever the order in
// which workgroups run.
//
// select_topk: one workgroup per live beam slot.  Candidates are the codes of the beam's
//   CSR trie row (or all C codes).  They stream through an LDS buffer; whenever it fills,
//   a radix select keeps the beam's top_k and raises the admission threshold, so a long
//   row costs one HBM read.  The survivors go to the request's pool (one atomic
//   reservation per workgroup).  A beam that alone holds >= W_r survivors publishes its
//   W_r-th best key as a lower bound of the request's W_r-th best; beams whose score is
//   below that bound exit without reading their row (log-probabilities are <= 0, so no
//   key exceeds its beam's score), and candidates below it are never buffered.
// select_global: one workgroup per request: radix select of the W_r-th best pool entry,
//   gather, bitonic sort in LDS, then the outputs (the exact float32 score is recomputed
//   from its two operands, the trie child by a binary search of the parent's row).
//   It leaves the pool counter and the bound at zero for the next step.
#include "device_common.h"
#include "grw_internal.h"

namespace grw {

namespace {

// Threshold T such that exactly N of the n distinct entries get(0..n-1) are >= T
// (1 <= N <= n): most-significant-digit-first radix select, 8-bit digits, histograms in
// LDS, stopping as soon as the chosen digit's bucket holds exactly the entries still
// needed.
template <int NT, typename Get>
__device__ uint64_t block_select_threshold(Get get, int n, int N, uint32_t* hist, uint32_t* scr) {
  uint64_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)N;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint64_t v = get(i);
      if ((v & mask) == prefix) atomicAdd(&hist[(uint32_t)(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const uint32_t c0 = hist[255 - 4 * lane], c1 = hist[254 - 4 * lane];
      const uint32_t c2 = hist[253 - 4 * lane], c3 = hist[252 - 4 * lane];
      const uint32_t tot = c0 + c1 + c2 + c3;
      const uint32_t incl = (uint32_t)wave_inclusive_scan((int)tot);
      const uint32_t excl = incl - tot;
      if (excl < need && need <= incl) {
        uint32_t acc = excl;
        int dsel;
        if (acc + c0 >= need) dsel = 255 - 4 * lane;
        else if ((acc += c0) + c1 >= need) dsel = 254 - 4 * lane;
        else if ((acc += c1) + c2 >= need) dsel = 253 - 4 * lane;
        else { acc += c2; dsel = 252 - 4 * lane; }
        scr[0] = (uint32_t)dsel;
        scr[1] = acc;
        scr[2] = hist[dsel];
      }
    }
    __syncthreads();
    const uint32_t dsel = scr[0], above = scr[1], cnt = scr[2];
    __syncthreads();
    need -= above;
    prefix |= (uint64_t)dsel << shift;
    mask |= (uint64_t)255u << shift;
    if (cnt == need) return prefix;
  }
  return prefix;
}

// Append each thread's `ne` entries (registers) to dst[*counter ...] (LDS counter).
// Must be reached by every thread of the workgroup.
template <int NE>
__device__ __forceinline__ void block_append(uint64_t* dst, int* counter, const uint64_t (&e)[NE], int ne) {
  const int lane = threadIdx.x & 63;
  const int incl = wave_inclusive_scan(ne);
  const int total = __shfl(incl, 63, 64);
  int base = 0;
  if (lane == 63 && total > 0) base = atomicAdd(counter, total);
  base = __shfl(base, 63, 64);
  const int pos = base + incl - ne;
#pragma unroll
  for (int k = 0; k < NE; ++k)
    if (k < ne) dst[pos + k] = e[k];
}

// Keep only entries >= T of buf[0..n) (in LDS), compacted to the front; returns the new n.
__device__ int block_compact_ge(uint64_t* buf, int n, uint64_t T, int* counter) {
  constexpr int PER = kSelCap / 256;   // 16 entries per thread
  uint64_t v[PER];
  int nv = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i < n) {
      const uint64_t x = buf[i];
      if (x >= T) v[nv++] = x;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) *counter = 0;
  __syncthreads();
  block_append<PER>(buf, counter, v, nv);
  __syncthreads();
  return *counter;
}

__global__ __launch_bounds__(256) void select_topk_kernel(SelArgs a) {
  __shared__ uint64_t buf[kSelCap];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scr[4];
  __shared__ int cnt_s;
  __shared__ int flag_s;
  __shared__ uint32_t pos_s;
  const int slot = blockIdx.x;
  const int tid = threadIdx.x;
  const float s = a.scores[slot];
  if (s == -INFINITY) return;
  if (__builtin_isnan(s)) {
    if (tid == 0) atomicOr(a.flags, (int)GRW_FLAG_NAN_LOGPROB);
    return;
  }
  const int r = a.slot_req[slot];
  const ReqDesc rd = a.req[r];
  const uint32_t s_key = ordered_key(s);
  // one read of the request's bound, shared by the workgroup so the exit is uniform
  if (tid == 0) pos_s = __hip_atomic_load(&a.bound[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  uint32_t tau = pos_s;
  if (s_key < tau) return;                       // early exit: no key of this beam can make it

  int cnt = a.C;
  const int32_t* codes = nullptr;
  if (a.row_ptr != nullptr) {
    const int node = a.nodes[slot];
    if (node < 0 || node >= a.n_internal) {
      if (tid == 0) atomicOr(a.flags, (int)GRW_FLAG_BAD_NODE);
      return;
    }
    const int beg = a.row_ptr[node];
    cnt = a.row_ptr[node + 1] - beg;
    codes = a.code + beg;
  }
  const float* lprow = a.logprobs + (size_t)slot * a.C;
  const uint32_t flat_base = (uint32_t)(slot - rd.boff) * (uint32_t)a.C;
  const int K = rd.K;
  if (tid == 0) { cnt_s = 0; flag_s = 0; }
  __syncthreads();

  int n = 0;
  int fl = 0;
  for (int base = 0; base < cnt; base += kSelChunk) {
    if (n + kSelChunk > kSelCap) {               // buffer full: keep the top K, raise tau
      const uint64_t T = block_select_threshold<256>([&](int i) { return buf[i]; }, n, K, hist, scr);
      n = block_compact_ge(buf, n, T, &cnt_s);
      const uint32_t tk = (uint32_t)(T >> 32);
      tau = max(tau, tk);
      tau = max(tau, __hip_atomic_load(&a.bound[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
    uint64_t e[4];
    int ne = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = base + tid + 256 * k;
      if (i < cnt) {
        const int c = codes ? codes[i] : i;
        if ((unsigned)c >= (unsigned)a.C) {        // corrupt trie row: never read outside the row
          fl |= GRW_FLAG_BAD_NODE;
          continue;
        }
        const float lp = lprow[c];
        if (__builtin_isnan(lp)) {
          fl |= GRW_FLAG_NAN_LOGPROB;
        } else {
          if (lp > 0.0f) fl |= GRW_FLAG_POS_LOGPROB;
          const float key = s + lp;
          if (key != -INFINITY) {
            const uint32_t ok = ordered_key(key);
            if (ok >= tau) e[ne++] = composite_key(ok, flat_base + (uint32_t)c);
          }
        }
      }
    }
    block_append<4>(buf, &cnt_s, e, ne);
    __syncthreads();
    n = cnt_s;
  }
  if (fl) atomicOr(&flag_s, fl);

  // survivors: the top min(n, K) entries
  uint64_t T = 0;
  int n_surv = n;
  if (n > K) {
    T = block_select_threshold<256>([&](int i) { return buf[i]; }, n, K, hist, scr);
    n_surv = K;
  }
  if (n_surv > 0) {
    // lower bound of the request's W-th best key: this beam's own W-th best survivor
    if (n_surv >= rd.W) {
      uint64_t TW;
      if (n_surv == rd.W && n > K) TW = T;
      else TW = block_select_threshold<256>([&](int i) { return buf[i]; }, n, rd.W, hist, scr);
      if (tid == 0) atomicMax(&a.bound[r], (uint32_t)(TW >> 32));
    }
    if (tid == 0) pos_s = atomicAdd(&a.pool_count[r], (uint32_t)n_surv);
    __syncthreads();
    uint64_t* dst = a.pool + rd.pool_off + pos_s;
    if (tid == 0) cnt_s = 0;
    __syncthreads();
    for (int base = 0; base < n; base += 1024) {
      uint64_t e[4];
      int ne = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = base + tid + 256 * k;
        if (i < n && buf[i] >= T) e[ne++] = buf[i];
      }
      block_append<4>(dst, &cnt_s, e, ne);
    }
  }
  __syncthreads();
  if (tid == 0 && flag_s) atomicOr(a.flags, flag_s);
}

__global__ __launch_bounds__(1024) void select_global_kernel(SelArgs a) {
  __shared__ uint64_t sel[kMaxW];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scr[4];
  __shared__ int cnt_s;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const ReqDesc rd = a.req[r];
  const int n = (int)a.pool_count[r];
  const uint64_t* pool = a.pool + rd.pool_off;
  const int W = rd.W;
  const int nsel = min(n, W);
  uint64_t T = 0;
  if (n > W) T = block_select_threshold<1024>([&](int i) { return pool[i]; }, n, W, hist, scr);
  if (tid == 0) cnt_s = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + tid;
    uint64_t e[1];
    int ne = 0;
    if (i < n) {
      const uint64_t v = pool[i];
      if (v >= T) e[ne++] = v;
    }
    block_append<1>(sel, &cnt_s, e, ne);
  }
  __syncthreads();
  int npow = 1;
  while (npow < nsel) npow <<= 1;
  for (int i = nsel + tid; i < npow; i += 1024) sel[i] = 0ull;   // sorts last
  __syncthreads();
  for (int k = 2; k <= npow; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < npow; i += 1024) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = sel[i], y = sel[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            sel[i] = y;
            sel[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  const int C = a.C;
  for (int i = tid; i < W; i += 1024) {
    const int slot = rd.boff + i;
    if (i < nsel) {
      const uint32_t flat = composite_flat(sel[i]);
      const uint32_t b = flat / (uint32_t)C;
      const int c = (int)(flat - b * (uint32_t)C);
      const int ps = rd.boff + (int)b;
      const float score = a.scores[ps] + a.logprobs[(size_t)ps * C + c];
      int node = -1;
      if (a.row_ptr != nullptr) {
        const int pn = a.nodes[ps];
        int lo = a.row_ptr[pn], hi = a.row_ptr[pn + 1] - 1;
        node = -1;
        while (lo <= hi) {
          const int mid = (lo + hi) >> 1;
          const int cm = a.code[mid];
          if (cm == c) { node = mid + 1; break; }
          if (cm < c) lo = mid + 1; else hi = mid - 1;
        }
        if (node < 0) atomicOr(a.flags, (int)GRW_FLAG_CHILD_MISSING);
      }
      a.out_token[slot] = c;
      a.out_parent[slot] = (int)b;
      a.out_score[slot] = score;
      a.out_node[slot] = node;
    } else {
      a.out_token[slot] = -1;
      a.out_parent[slot] = -1;
      a.out_score[slot] = -INFINITY;
      a.out_node[slot] = -1;
    }
  }
  __syncthreads();
  if (tid == 0) {
    a.pool_count[r] = 0u;
    a.bound[r] = 0u;
  }
}

__global__ void beams_init_kernel(const ReqDesc* req, const int32_t* slot_req, int sumW,
                                  float* scores, int32_t* nodes) {
  const int slot = blockIdx.x * 256 + threadIdx.x;
  if (slot >= sumW) return;
  const bool first = slot == req[slot_req[slot]].boff;
  scores[slot] = first ? 0.0f : -INFINITY;
  nodes[slot] = first ? 0 : -1;
}

__global__ void backtrack_kernel(const ReqDesc* req, const int32_t* slot_req, int sumW,
                                 const int32_t* tokens, const int32_t* parents, int S, int32_t* sid) {
  const int slot = blockIdx.x * 256 + threadIdx.x;
  if (slot >= sumW) return;
  const ReqDesc rd = req[slot_req[slot]];
  int j = slot - rd.boff;
  bool pad = false;
  for (int d = S - 1; d >= 0; --d) {
    const int gs = rd.boff + j;
    const int t = tokens[(size_t)d * sumW + gs];
    if (t < 0) { pad = true; break; }
    sid[(size_t)slot * S + d] = t;
    if (d > 0) {
      j = parents[(size_t)d * sumW + gs];
      if (j < 0 || j >= rd.W) { pad = true; break; }
    }
  }
  if (pad)
    for (int d = 0; d < S; ++d) sid[(size_t)slot * S + d] = -1;
}

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_select_topk(const SelArgs& a, hipStream_t s) {
  if (a.sumW == 0) return hipSuccess;
  select_topk_kernel<<<a.sumW, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_select_global(const SelArgs& a, hipStream_t s) {
  if (a.R == 0) return hipSuccess;
  select_global_kernel<<<a.R, 1024, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_beams_init(const ReqDesc* req, const int32_t* slot_req, int32_t sumW,
                             float* scores, int32_t* nodes, hipStream_t s) {
  if (sumW == 0) return hipSuccess;
  beams_init_kernel<<<(sumW + 255) / 256, 256, 0, s>>>(req, slot_req, sumW, scores, nodes);
  return hipGetLastError();
}

hipError_t launch_backtrack(const ReqDesc* req, const int32_t* slot_req, int32_t sumW,
                            const int32_t* tokens, const int32_t* parents, int32_t S,
                            int32_t* sid, hipStream_t s) {
  if (sumW == 0) return hipSuccess;
  backtrack_kernel<<<(sumW + 255) / 256, 256, 0, s>>>(req, slot_req, sumW, tokens, parents, S, sid);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  zero_u32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace grw
