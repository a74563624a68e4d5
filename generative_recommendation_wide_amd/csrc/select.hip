// Beam selection (xLLM generative-recommendation design doc, section 4.1.1: each beam
// expands top_k candidates, the next beam set is the best beam_width of the
// beam_width x top_k pool; section 4.3: stop unnecessary sorting early, filter invalid
// item paths early, reuse candidate containers; FlashRec announcement: with the fused
// semantic-ID trie illegal IDs are never candidates).
//
// Keys are compared as 64-bit composites (order-preserving float key, ~flat index), so one
// unsigned comparison orders by (key descending, flat index ascending) and every
// candidate is distinct: the selection is unique and deterministic whatever the order in
// which workgroups run.  A composite of a real candidate is never 0, so 0 marks "empty".
//
// Kernels per step:
//
// select_pilot / select_bound: the first few slots of each request (the best beams of the
//   previous step) are pilots.  Each pilot contributes one candidate per group of threads,
//   at most top_k of them; the W_r-th best of a request's contributions is a lower bound of
//   its W_r-th best pool entry, because a pilot beam's i-th best contribution is at most
//   its i-th best candidate and its top_k candidates are all in the pool.
// select_topk: one workgroup per beam slot; each writes its survivors to its own region of
//   the request's pool (no shared counters).  A beam whose score is below the bound keeps
//   nothing and reads nothing: log-probabilities are <= 0, so no key exceeds its beam's
//   score.  Rows of up to 8192 candidates are read once into registers; candidates below
//   the bound are dropped, and a radix select over the registers keeps the beam's top_k
//   when more remain.  Longer rows stream through an LDS buffer that a radix select trims
//   to top_k whenever it fills.  A beam that alone holds >= W_r survivors raises the bound
//   to its own W_r-th best.
// On the register-resident path (rows of at most 8192 codes, W <= 1024) the pilots and the
// per-beam stage share one launch (select_pilot_beam): the pilots are its first
// workgroups, and the beam workgroups read their rows at once and wait for the bound, which
// the request's last pilot publishes in a step word; the W-of-pool stage follows as
// select_final.
// select_global: one workgroup per request.  The beams' survivor counts give every entry a
//   place in one index range.  A histogram of the entries' keys (bins measured down from
//   the best live score) finds the bin that holds the W_r-th best entry; the entries of
//   that bin and all better bins are placed bin by bin and ranked inside their bin, which
//   gives every winner its output position directly.  When a bin is too large to rank in
//   place, a radix select and a bitonic sort in LDS do the same job.  The outputs carry the
//   exact float32 score (recomputed from its two operands) and the trie child (binary
//   search of the parent's row).  The kernel leaves the bound at zero for the next step.
#include "device_common.h"
#include "grw_internal.h"

namespace grw {

namespace {

// hist[d] += 1 for every active lane with `on` set.  The lanes whose digit equals that of
// the wave's first such lane are counted with one atomic, the others one by one.  Used for
// a radix select's first digit when that digit lies in the sign and exponent bits of an
// ordered float key: such digits cluster in one or two values (three quarters of a
// log-probability row's 8192 keys share one), and same-address LDS atomics of one
// instruction serialise.  Mantissa digits are spread, and there the extra ballots and the
// second atomic cost several times what they save.  Divergence-safe (the lane masks cover
// the active lanes only).
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t d, bool on) {
  const uint64_t act = __ballot(on);
  if (act == 0) return;
  const int first = __builtin_ctzll(act);
  const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)d, first);
  const bool same = on && d == d0;
  const uint64_t m = __ballot(same);
  if ((int)(threadIdx.x & 63) == first) atomicAdd(&hist[d0], (uint32_t)__popcll(m));
  else if (on && !same) atomicAdd(&hist[d], 1u);
}

// Pick, from a 256-bucket histogram, the digit whose bucket holds the `need`-th largest
// entry (buckets scanned from digit 255 down).  Run by the first wave; writes the digit,
// the count of entries in higher buckets and the bucket's own count to scr[0..2].
__device__ __forceinline__ void pick_digit(const uint32_t* hist, uint32_t need, uint32_t* scr) {
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

// Threshold T such that exactly N of the non-zero entries among get(0..n-1) are >= T
// (1 <= N <= their count; entries distinct): most-significant-digit-first radix select,
// 8-bit digits, histograms in LDS, stopping as soon as the chosen digit's bucket holds
// exactly the entries still needed.
template <int NT, typename Get>
__device__ __forceinline__ uint64_t block_select_threshold(Get get, int n, int N, uint32_t* hist, uint32_t* scr) {
  uint64_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)N;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint64_t v = get(i);
      const bool on = v != 0 && (v & mask) == prefix;
      if (mask == 0) hist_add(hist, (uint32_t)(v >> shift) & 255u, on);
      else if (on) atomicAdd(&hist[(uint32_t)(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) pick_digit(hist, need, scr);
    __syncthreads();
    const uint32_t dsel = scr[0], above = scr[1], cnt = scr[2];
    __syncthreads();
    need -= above;
    prefix |= (uint64_t)dsel << shift;
    mask |= (uint64_t)255u << shift;
    if (cnt == need) return prefix > 0 ? prefix : 1;
  }
  return prefix;
}

// Block-wide OR and AND of the threads' values (NT threads; red holds 2 NT / 64 entries).
template <int NT>
__device__ __forceinline__ void block_or_and(uint64_t& o, uint64_t& an, uint64_t* red) {
  constexpr int NW = NT / 64;
  o = wave_butterfly(o, [](uint64_t x, uint64_t y) { return x | y; });
  an = wave_butterfly(an, [](uint64_t x, uint64_t y) { return x & y; });
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { red[wave] = o; red[NW + wave] = an; }
  __syncthreads();
  o = 0;
  an = ~0ull;
#pragma unroll
  for (int w = 0; w < NW; ++w) { o |= red[w]; an &= red[NW + w]; }
}

// Sum over the 256 threads of a workgroup; red holds 4 entries.
__device__ __forceinline__ int block_sum256(int v, int* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Exclusive prefix of v over the 256 threads; *total receives the sum.  red holds 4 entries.
__device__ __forceinline__ int block_excl_scan256(int v, int* red, int* total) {
  const int incl = wave_inclusive_scan(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = incl;
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  int before = 0;
  for (int w = 0; w < wave; ++w) before += red[w];
  *total = red[0] + red[1] + red[2] + red[3];
  return before + incl - v;
}

// Exclusive prefix of v over the NT threads; *total receives the sum.  red holds NT / 64
// entries.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* red, int* total) {
  constexpr int NW = NT / 64;
  const int incl = wave_inclusive_scan(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = incl;
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) before += red[w];
    all += red[w];
  }
  *total = all;
  return before + incl - v;
}

// Threshold T such that exactly N of the non-zero entries held by the threads are >= T
// (1 <= N <= their count; NT threads, each holding NR entries get(0..NR-1), 0 = none).
// Radix select as above, starting at the highest bit in which the entries differ.
template <int NT, int NR, typename Get>
__device__ __forceinline__ uint64_t regs_select_threshold(Get get, int N, uint32_t* hist, uint32_t* scr,
                                                          uint64_t* red) {
  uint64_t o = 0, an = ~0ull;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const uint64_t x = get(k);
    if (x) { o |= x; an &= x; }
  }
  block_or_and<NT>(o, an, red);
  const uint64_t diff = o ^ an;
  if (diff == 0) return o;                         // a single distinct entry
  const int hb = 63 - __builtin_clzll(diff);
  const uint64_t below = (hb == 63) ? ~0ull : ((1ull << (hb + 1)) - 1);
  uint64_t known = ~below;
  uint64_t prefix = o & known;
  uint32_t need = (uint32_t)N;
  int shift = hb >= 7 ? hb - 7 : 0;
  for (bool first = true;; first = false) {
    for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const uint64_t x = get(k);
      const bool on = x != 0 && (x & known) == prefix;
      if (first && shift >= 55) hist_add(hist, (uint32_t)(x >> shift) & 255u, on);
      else if (on) atomicAdd(&hist[(uint32_t)(x >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) pick_digit(hist, need, scr);
    __syncthreads();
    const uint32_t dsel = scr[0], above = scr[1], cnt = scr[2];
    __syncthreads();
    need -= above;
    prefix |= (uint64_t)dsel << shift;
    known |= (uint64_t)255u << shift;
    if (cnt == need || shift == 0) return prefix > 0 ? prefix : 1;
    shift = shift >= 8 ? shift - 8 : 0;
  }
}

// 32-bit radix select over the non-zero values held by the threads (NT threads, NR values
// get(0..NR-1) each, n of them non-zero in total, 1 <= N <= n).  Returns v, need and cnt:
// exactly N - need values exceed v, and cnt values lie in [v, v + span) where span covers
// the bits not yet examined; cnt == need means the values >= v are exactly N, otherwise all
// 32 bits are examined and cnt values equal v, of which `need` are wanted.
struct Sel32 { uint32_t v, need, cnt; };

template <int NT, int NR, typename Get>
__device__ __forceinline__ Sel32 regs_select32(Get get, uint32_t N, uint32_t n, uint32_t* hist, uint32_t* scr,
                                               uint32_t* red) {
  constexpr int NW = NT / 64;
  uint32_t o = 0, an = ~0u;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const uint32_t x = get(k);
    if (x) { o |= x; an &= x; }
  }
  o = wave_butterfly(o, [](uint32_t x, uint32_t y) { return x | y; });
  an = wave_butterfly(an, [](uint32_t x, uint32_t y) { return x & y; });
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { red[threadIdx.x >> 6] = o; red[NW + (threadIdx.x >> 6)] = an; }
  __syncthreads();
  o = 0;
  an = ~0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) { o |= red[w]; an &= red[NW + w]; }
  const uint32_t diff = o ^ an;
  if (diff == 0) return Sel32{o, N, n};            // all values equal
  const int hb = 31 - __builtin_clz(diff);
  const uint32_t below = hb == 31 ? ~0u : ((1u << (hb + 1)) - 1);
  uint32_t known = ~below;
  uint32_t prefix = o & known;
  uint32_t need = N;
  int shift = hb >= 7 ? hb - 7 : 0;
  for (bool first = true;; first = false) {
    for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const uint32_t x = get(k);
      const bool on = x != 0 && (x & known) == prefix;
      if (first && shift >= 23) hist_add(hist, (x >> shift) & 255u, on);
      else if (on) atomicAdd(&hist[(x >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) pick_digit(hist, need, scr);
    __syncthreads();
    const uint32_t dsel = scr[0], above = scr[1], cnt = scr[2];
    __syncthreads();
    need -= above;
    prefix |= dsel << shift;
    known |= 255u << shift;
    if (cnt == need || shift == 0) return Sel32{prefix, need, cnt};
    shift = shift >= 8 ? shift - 8 : 0;
  }
}

// Composite threshold T such that exactly N of the candidates held by the threads are
// >= T, from their ordered keys ok(k) (0 = none) and flat indices flat(k); n candidates in
// all.  Ties at the threshold key are resolved by a second select on ~flat.
template <int NT, int NR, typename GetKey, typename GetFlat>
__device__ __forceinline__ uint64_t regs_select_composite(GetKey ok, GetFlat flat, uint32_t N, uint32_t n,
                                                          uint32_t* hist, uint32_t* scr, uint32_t* red) {
  const Sel32 t = regs_select32<NT, NR>(ok, N, n, hist, scr, red);
  if (t.cnt == t.need) return (uint64_t)t.v << 32;
  const Sel32 t2 = regs_select32<NT, NR>([&](int k) { return ok(k) == t.v ? ~flat(k) : 0u; }, t.need, t.cnt, hist,
                                         scr, red);
  return ((uint64_t)t.v << 32) | t2.v;
}

// Append each thread's `ne` entries (registers) to dst[*counter ...] (LDS counter).
// Must be reached by every thread of the workgroup.
template <int NE>
__device__ __forceinline__ void block_append(uint64_t* dst, int* counter, const uint64_t (&e)[NE], int ne) {
  const int lane = threadIdx.x & 63;
  const int incl = wave_inclusive_scan(ne);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  int base = 0;
  if (lane == 63 && total > 0) base = atomicAdd(counter, total);
  base = __builtin_amdgcn_readlane(base, 63);
  const int pos = base + incl - ne;
#pragma unroll
  for (int k = 0; k < NE; ++k)
    if (k < ne) dst[pos + k] = e[k];
}

// Keep only entries >= T of buf[0..n) (in LDS), compacted to the front; returns the new n.
__device__ __forceinline__ int block_compact_ge(uint64_t* buf, int n, uint64_t T, int* counter) {
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

// The candidates of a beam slot: its CSR trie row (or all C codes), and the node's dense
// child bit mask when the trie has one for it (FlashRec announcement: the SID trie is dense
// or CSR).  Returns false when the node is out of range.
__device__ __forceinline__ bool beam_row(const SelArgs& a, int slot, int& cnt, const int32_t*& codes,
                                         const uint32_t** mask = nullptr) {
  cnt = a.C;
  codes = nullptr;
  if (mask) *mask = nullptr;
  if (a.row_ptr != nullptr) {
    const int node = a.nodes[slot];
    if (node < 0 || node >= a.n_internal) return false;
    const int beg = a.row_ptr[node];
    cnt = a.row_ptr[node + 1] - beg;
    codes = a.code + beg;
    if (mask && a.dense_slot != nullptr) {
      const int ds = a.dense_slot[node];
      if (ds >= 0) *mask = a.dense_mask + (size_t)ds * a.mask_words;
    }
  }
  return true;
}

// Gumbel top-k (FlashRec deployment guide, request section: a positive temperature orders
// the candidates by a Gumbel-perturbed key, the returned score holds no noise).  With noise
// (G), the ordering key of a candidate is fl32(key + tg) with tg = fl32(T * g), each an
// IEEE rounding of its own (no fused multiply-add).  tg of one candidate:
__device__ __forceinline__ float noise_term(const SelArgs& a, const float* grow, int c, int& fl) {
  const float g = grow[c];
  if (!__builtin_isfinite(g)) fl |= GRW_FLAG_BAD_NOISE;
  return __fmul_rn(a.temp, g);
}

// The ordering key from the key and tg (the key itself without noise).
template <bool G>
__device__ __forceinline__ float order_key(float key, float tg) {
  if constexpr (G) return __fadd_rn(key, tg);
  else return key;
}

// Composite key of one candidate (0 when it is not a candidate), with the precondition flags.
template <bool G>
__device__ __forceinline__ uint64_t candidate(float s, float lp, float tg, uint32_t flat, int& fl) {
  if (__builtin_isnan(lp)) { fl |= GRW_FLAG_NAN_LOGPROB; return 0; }
  if (lp > 0.0f) fl |= GRW_FLAG_POS_LOGPROB;
  const float key = s + lp;
  if (key == -INFINITY) return 0;
  const float ok = order_key<G>(key, tg);
  if (ok == -INFINITY || __builtin_isnan(ok)) return 0;
  return composite_key(ordered_key(ok), flat);
}

// Selection from raw logits (the fused log-softmax): the log-softmax of a row of C logits
// is lp = fl32(x - lse) with lse = fl32(ln sum exp(x)) over the whole row, the sum taken in
// float64 after subtracting the row max.  Every row's lse is computed once, by one
// workgroup, and kept in row_lse for the kernels that read the row again.
//
// lse of the row whose values the NT threads hold in v (-inf outside the row), with the
// precondition flag for NaN or +inf logits.  redf holds NT / 64 floats, redd NT / 64 doubles.
template <int NT, int N>
__device__ __forceinline__ float block_lse(const float (&v)[N], float* redf, double* redd, int& fl) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float m = -INFINITY;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    bad |= __builtin_isnan(v[k]) || v[k] == INFINITY;
    m = fmaxf(m, v[k]);
  }
  if (bad) fl |= GRW_FLAG_NAN_LOGPROB;
  m = wave_max(m);
  __syncthreads();
  if (lane == 0) redf[wave] = m;
  __syncthreads();
  m = redf[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmaxf(m, redf[w]);
  double sum = 0.0;
  const double md = (double)m;
#pragma unroll
  for (int k = 0; k < N; ++k) sum += exp((double)v[k] - md);    // exp(-inf) = 0
  sum = wave_sum(sum);
  if (lane == 0) redd[wave] = sum;
  __syncthreads();
  sum = redd[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) sum += redd[w];
  return (float)(md + log(sum));
}

// lse of a full row of C logits read with stride 256 (rows of at most kOnePass codes).
__device__ __forceinline__ float row_lse_strided(const float* xrow, int C, float* redf, double* redd, int& fl) {
  float v[kRegC];
#pragma unroll
  for (int k = 0; k < kRegC; ++k) {
    const int i = (int)threadIdx.x + 256 * k;
    v[k] = i < C ? xrow[i] : -INFINITY;
  }
  return block_lse<256, kRegC>(v, redf, redd, fl);
}

// Row layouts of the one-read path: kFull — all C codes with C % 4 == 0 and an aligned row,
// thread t holding codes 4 (t + 256 q) + e so that every load is a full 1 KB wave line;
// kFullScalar — all C codes, thread t holding codes t + 256 k; kTrie — a CSR trie row,
// thread t holding row positions t + 256 k (their codes are kept).
enum RowLayout { kFull = 0, kFullScalar = 1, kTrie = 2 };

template <int L, bool G = false>
struct RowRegs {
  float lp[kRegC];
  float tg[G ? kRegC : 1];     // fl32(T * g) of each position (sampled selection)
  int code[L == kTrie ? kRegC : 1];
  __device__ __forceinline__ int code_of(int k) const {
    if constexpr (L == kTrie) return code[k];
    else if constexpr (L == kFull) return 4 * ((int)threadIdx.x + 256 * (k >> 2)) + (k & 3);
    else return (int)threadIdx.x + 256 * k;
  }
  __device__ __forceinline__ bool valid(int k, int cnt) const {
    if constexpr (L == kTrie) return code[k] >= 0;
    else return code_of(k) < cnt;
  }
};

// Read a row of up to kOnePass candidates into registers (one load per candidate), and with
// noise (G) the noise terms of the same positions from grow.  Positions that hold no
// candidate read as -inf.
template <int L, bool G = false>
__device__ __forceinline__ void load_row(RowRegs<L, G>& rr, const SelArgs& a, const float* lprow,
                                         const float* grow, const int32_t* codes, int cnt, int& fl,
                                         const uint32_t* mask = nullptr) {
  const int tid = threadIdx.x;
  if constexpr (L == kTrie) {
    if (mask != nullptr) {
      // dense row: thread t holds codes t + 256 k, read in full lines; the bit mask keeps the
      // children (a wave's 64 codes of one k share two mask words)
#pragma unroll
      for (int k = 0; k < kRegC; ++k) {
        const int c = tid + 256 * k;
        const bool ok = c < a.C && ((mask[c >> 5] >> (c & 31)) & 1u);
        rr.code[k] = ok ? c : -1;
        rr.lp[k] = ok ? lprow[c] : -INFINITY;
        if constexpr (G) rr.tg[k] = ok ? noise_term(a, grow, c, fl) : 0.0f;
      }
      return;
    }
  }
  if constexpr (L == kFull) {
#pragma unroll
    for (int q = 0; q < kRegC / 4; ++q) {
      const int i = 4 * (tid + 256 * q);
      floatx4 x, y;
      if (i + 3 < cnt) {
        x = *(const floatx4*)(lprow + i);
        if constexpr (G) y = *(const floatx4*)(grow + i);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = i + e < cnt ? lprow[i + e] : -INFINITY;
          if constexpr (G) y[e] = i + e < cnt ? grow[i + e] : 0.0f;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rr.lp[4 * q + e] = x[e];
        if constexpr (G) {
          if (!__builtin_isfinite(y[e])) fl |= GRW_FLAG_BAD_NOISE;
          rr.tg[4 * q + e] = __fmul_rn(a.temp, y[e]);
        }
      }
    }
  } else if constexpr (L == kFullScalar) {
#pragma unroll
    for (int k = 0; k < kRegC; ++k) {
      const int i = tid + 256 * k;
      rr.lp[k] = i < cnt ? lprow[i] : -INFINITY;
      if constexpr (G) rr.tg[k] = i < cnt ? noise_term(a, grow, i, fl) : 0.0f;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kRegC; ++k) {
      const int i = tid + 256 * k;
      rr.code[k] = i < cnt ? codes[i] : -1;
    }
#pragma unroll
    for (int k = 0; k < kRegC; ++k) {
      const bool in_row = tid + 256 * k < cnt;
      const bool ok = in_row && (unsigned)rr.code[k] < (unsigned)a.C;
      if (in_row && !ok) fl |= GRW_FLAG_BAD_NODE;   // corrupt trie row: never read outside the row
      rr.lp[k] = ok ? lprow[rr.code[k]] : -INFINITY;
      if constexpr (G) rr.tg[k] = ok ? noise_term(a, grow, rr.code[k], fl) : 0.0f;
      if (!ok) rr.code[k] = -1;
    }
  }
}

// Raw logits loaded into rr.lp -> log-probabilities: the row's lse is computed here (from
// the registers when they hold the whole row, else from a strided pass over it) and stored
// in row_lse, or, when another kernel already computed it, read from row_lse.  Reached by
// every thread of the workgroup.
template <int L, bool G>
__device__ __forceinline__ void to_logprobs(RowRegs<L, G>& rr, const SelArgs& a, int slot, const float* xrow,
                                            bool compute, float* redf, double* redd, int& fl) {
  float lse;
  if (compute) {
    if constexpr (L == kTrie) lse = row_lse_strided(xrow, a.C, redf, redd, fl);
    else lse = block_lse<256, kRegC>(rr.lp, redf, redd, fl);
    if (threadIdx.x == 0) a.row_lse[slot] = lse;
  } else {
    lse = a.row_lse[slot];
  }
#pragma unroll
  for (int k = 0; k < kRegC; ++k) rr.lp[k] = rr.lp[k] - lse;     // -inf stays -inf
}

// Ordered key of candidate k of a loaded row (0 when it is not a candidate or is below
// tau), with the precondition flags.
template <int L, bool G>
__device__ __forceinline__ uint32_t row_key(const RowRegs<L, G>& rr, int k, int cnt, float s, uint32_t tau, int& fl) {
  if (!rr.valid(k, cnt)) return 0u;
  const float lp = rr.lp[k];
  if (__builtin_isnan(lp)) { fl |= GRW_FLAG_NAN_LOGPROB; return 0u; }
  if (lp > 0.0f) fl |= GRW_FLAG_POS_LOGPROB;
  const float key = s + lp;
  if (key == -INFINITY) return 0u;
  const float okf = order_key<G>(key, G ? rr.tg[k] : 0.0f);
  if (okf == -INFINITY || __builtin_isnan(okf)) return 0u;
  const uint32_t o = ordered_key(okf);
  return o >= tau ? o : 0u;
}

// The best candidate of a loaded row of up to kOnePass candidates (0 when none).
template <int L, bool G, bool X>
__device__ __forceinline__ uint64_t loaded_row_best(RowRegs<L, G>& rr, const SelArgs& a, int slot, const float* lprow,
                                                    int cnt, float s, uint32_t flat_base, int& fl, float* redf,
                                                    double* redd) {
  if constexpr (X) to_logprobs<L, G>(rr, a, slot, lprow, a.lse_ready == 0, redf, redd, fl);
  if constexpr (L == kTrie) {
    uint64_t best = 0;
#pragma unroll
    for (int k = 0; k < kRegC; ++k) {
      const uint32_t o = row_key<L>(rr, k, cnt, s, 0u, fl);
      if (o) best = max(best, composite_key(o, flat_base + (uint32_t)rr.code_of(k)));
    }
    return best;
  } else {
    // full rows: a thread's codes rise with k, so the largest composite is the largest
    // ordered key at the smallest k that holds it
    uint32_t ok[kRegC];
    uint32_t om = 0u;
#pragma unroll
    for (int k = 0; k < kRegC; ++k) {
      ok[k] = row_key<L>(rr, k, cnt, s, 0u, fl);
      om = max(om, ok[k]);
    }
    int kb = 0;
#pragma unroll
    for (int k = kRegC - 1; k >= 0; --k) kb = ok[k] == om ? k : kb;
    return om ? composite_key(om, flat_base + (uint32_t)rr.code_of(kb)) : 0ull;
  }
}

// The best candidate of a row of up to kOnePass candidates (0 when none).
template <int L, bool G, bool X>
__device__ __forceinline__ uint64_t row_best(const SelArgs& a, int slot, const float* lprow, const float* grow,
                                             const int32_t* codes, int cnt, float s, uint32_t flat_base, int& fl,
                                             float* redf, double* redd, const uint32_t* mask = nullptr) {
  RowRegs<L, G> rr;
  load_row<L, G>(rr, a, lprow, grow, codes, cnt, fl, mask);
  if constexpr (X) to_logprobs<L, G>(rr, a, slot, lprow, a.lse_ready == 0, redf, redd, fl);
  uint64_t best = 0;
#pragma unroll
  for (int k = 0; k < kRegC; ++k) {
    const uint32_t o = row_key<L>(rr, k, cnt, s, 0u, fl);
    if (o) best = max(best, composite_key(o, flat_base + (uint32_t)rr.code_of(k)));
  }
  return best;
}

// The row layout of a beam's one-read path.
__device__ __forceinline__ int row_layout(const SelArgs& a, const int32_t* codes, const float* lprow) {
  if (codes != nullptr) return kTrie;
  const bool aligned = (((uintptr_t)lprow) & 15) == 0 &&
                       (a.noise == nullptr || ((((uintptr_t)a.noise) + (uintptr_t)(lprow - a.logprobs) * 4) & 15) == 0);
  return ((a.C & 3) == 0 && aligned) ? kFull : kFullScalar;
}

// Device-coherent access to data that another workgroup, possibly on another XCD, writes
// or reads during the same kernel (relaxed agent-scope atomics: no cache maintenance).
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this thread's stores are acknowledged at device scope
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup barrier that publishes LDS operations but leaves global loads in flight
// (__syncthreads also waits for every outstanding load, which would cancel a prefetch).
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Step-state word: bit 63 set once the request's bound (low 32 bits) is published.
constexpr uint64_t kSyncBound = 1ull << 63;

// Candidates a beam keeps: top_k, or at a first-step fan-out the request's beam width.  A
// fan-out wider than the per-beam selection holds (kMaxK) keeps every candidate instead,
// up to the request's whole pool region (W_r * K_r entries, at least the row length), and
// leaves the cut to W_r to the W-of-pool stage.
__device__ __forceinline__ int keep_k(const SelArgs& a, const ReqDesc& rd) {
  return !a.fanout ? rd.K : (rd.W <= kMaxK ? rd.W : rd.W * rd.K);
}
// Whether a slot expands: every slot, or at a first-step fan-out only the request's first.
__device__ __forceinline__ bool expands(const SelArgs& a, int slot, const ReqDesc& rd) {
  return !a.fanout || slot == rd.boff;
}

// --------------------------------------------------------------------------------------
// pilots and the request bound
// --------------------------------------------------------------------------------------
// One workgroup per pilot; descriptor {beam slot, request, first pilot-buffer entry,
// threads per group}.  Each pilot contributes one candidate per group of threads (at most
// top_k of its beam) with device-coherent stores and counts itself; the request's last
// pilot sets bound[r] to the W_r-th best key of all contributions (0 when there are fewer
// than W_r) and resets the count.
struct PilotLds {
  uint64_t red64[4];
  float redf[4];
  double redd[4];
  uint32_t hist[256];
  uint32_t scr[4];
  uint32_t red32[8];
  int red[4];
  int last;
};

// One contribution per group of pd.w threads of pilot pd (at most top_k per beam) goes to
// the pilot buffer; the pilot then counts itself in.  Returns true (in every thread) in the
// request's last pilot to count in.  Reached by every thread of the workgroup.
template <bool G, bool WIDE>
__device__ __forceinline__ bool pilot_contribute(const SelArgs& a, const int4 pd, const ReqDesc& rd, uint64_t best,
                                                 PilotLds& S) {
  uint64_t* red64 = S.red64;
  int& last_s = S.last;
  const int tid = threadIdx.x;
  const int r = pd.y, gsz = pd.w;
  // one contribution per group of gsz threads (at most top_k per beam)
  const int gl = gsz < 64 ? gsz : 64;
  if (gl > 1) best = max(best, lane_xor<1>(best));
  if (gl > 2) best = max(best, lane_xor<2>(best));
  if (gl > 4) best = max(best, lane_xor<4>(best));
  if (gl > 8) best = max(best, lane_xor<8>(best));
  if (gl > 16) best = max(best, lane_xor<16>(best));
  if (gl > 32) best = max(best, lane_xor<32>(best));
  if (gsz > 64) {
    if ((tid & 63) == 0) red64[tid >> 6] = best;
    __syncthreads();
    const int w0 = (tid >> 6) & ~((gsz >> 6) - 1);
    best = red64[w0];
    for (int w = 1; w < (gsz >> 6); ++w) best = max(best, red64[w0 + w]);
  }
  if (tid % gsz == 0) st_dev(&a.pilot_buf[pd.z + tid / gsz], best);
  wait_stores();
  __syncthreads();
  const int n_pilot = WIDE ? (G ? rd.n_pilot_ws : rd.n_pilot_w) : (G ? rd.n_pilot_s : rd.n_pilot);
  if (tid == 0) last_s = atomicAdd(&a.pilot_count[r], 1u) == (uint32_t)(n_pilot - 1);
  __syncthreads();
  return last_s;
}

// The request's last pilot: the W_r-th best key of all contributions bounds the request's
// W_r-th best pool entry.  PUBLISH: stored with a device-coherent store, then set in every
// copy of the request's step word.
template <bool G, bool PUBLISH, bool WIDE>
__device__ __forceinline__ void pilot_bound(const SelArgs& a, int r, int gsz, const ReqDesc& rd, PilotLds& S) {
  uint32_t* hist = S.hist;
  uint32_t* scr = S.scr;
  uint32_t* red32 = S.red32;
  int* red = S.red;
  const int tid = threadIdx.x;
  const int n_pilot = WIDE ? (G ? rd.n_pilot_ws : rd.n_pilot_w) : (G ? rd.n_pilot_s : rd.n_pilot);
  constexpr int NP = (WIDE ? kPilotCapWide : kPilotCap) / 256;
  const int n_ent = n_pilot * (256 / gsz);
  const uint64_t* pb = a.pilot_buf + rd.pilot_off;
  uint32_t pk[NP];
  int nv = 0;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int q = tid + 256 * k;
    pk[k] = q < n_ent ? (uint32_t)(ld_dev(&pb[q]) >> 32) : 0u;
    nv += pk[k] != 0u;
  }
  nv = block_sum256(nv, red);
  uint32_t lo = 0;
  if (nv >= rd.W)
    lo = regs_select32<256, NP>([&](int k) { return pk[k]; }, (uint32_t)rd.W, (uint32_t)nv, hist, scr, red32).v;
  if constexpr (PUBLISH) {
    // the bound in every copy of the step word, after the bound itself is stored for the
    // W-of-pool stage (beam workgroups raise it only after they have read the word)
    if (tid == 0) {
      st_dev(&a.bound[r], lo);
      st_dev(&a.pilot_count[r], 0u);
      wait_stores();
    }
    __syncthreads();
    if (tid < kSyncCopies)
      st_dev(&a.sync[((size_t)r * kSyncCopies + tid) * kSyncStride], kSyncBound | lo);
  } else if (tid == 0) {
    a.bound[r] = lo;
    a.pilot_count[r] = 0u;
  }
}

// Pilot workgroup `pi`.  PUBLISH (pilots inside the per-beam kernel): the request's last
// pilot stores the bound with a device-coherent store and, once that store is acknowledged,
// sets the request's ready word that the kernel's beam workgroups wait on.
// LT >= 0: every row of the launch has that layout and fits the one-read path.  WIDE: the
// general kernels' pilot set (up to kPilotCapWide contributions per request).
template <bool G, bool X, bool PUBLISH, int LT = -1, bool WIDE = false>
__device__ __forceinline__ void pilot_run(const SelArgs& a, int pi, PilotLds& S) {
  float* redf = S.redf;
  double* redd = S.redd;
  const int tid = threadIdx.x;
  const int4 pd = ((const int4*)a.pilot_desc)[pi];
  const int slot = pd.x, r = pd.y, gsz = pd.w;
  const float* lprow = a.logprobs + (size_t)slot * a.C;
  const float* grow = G ? a.noise + (size_t)slot * a.C : nullptr;
  int cnt = a.C, fl = 0;
  // full rows: the row loads go out before the descriptor loads (a dead beam's row is read
  // and ignored)
  constexpr bool kEarly = LT == kFull || LT == kFullScalar;
  RowRegs<kEarly ? LT : kFull, G> rr0;
  if constexpr (kEarly) load_row<LT, G>(rr0, a, lprow, grow, nullptr, cnt, fl);
  const ReqDesc rd = a.req[r];
  const float s = a.scores[slot];
  const uint32_t flat_base = (uint32_t)(slot - rd.boff) * (uint32_t)a.C;
  const int32_t* codes = nullptr;
  uint64_t best = 0;
  const uint32_t* mask = nullptr;
  if (s != -INFINITY && !__builtin_isnan(s) && expands(a, slot, rd) && beam_row(a, slot, cnt, codes, &mask)) {
    if constexpr (kEarly) {
      best = loaded_row_best<LT, G, X>(rr0, a, slot, lprow, cnt, s, flat_base, fl, redf, redd);
    } else if constexpr (LT >= 0) {
      if (cnt <= kOnePass) best = row_best<LT, G, X>(a, slot, lprow, grow, codes, cnt, s, flat_base, fl, redf, redd, mask);
    } else if (cnt <= kOnePass) {
      const int lay = row_layout(a, codes, lprow);
      if (lay == kFull) best = row_best<kFull, G, X>(a, slot, lprow, grow, codes, cnt, s, flat_base, fl, redf, redd);
      else if (lay == kFullScalar)
        best = row_best<kFullScalar, G, X>(a, slot, lprow, grow, codes, cnt, s, flat_base, fl, redf, redd);
      else best = row_best<kTrie, G, X>(a, slot, lprow, grow, codes, cnt, s, flat_base, fl, redf, redd, mask);
    } else {
      // long rows (lse computed by select_lse_kernel): 16 positions per thread per round,
      // their loads issued together
      const float lse = X ? a.row_lse[slot] : 0.0f;
      for (int q0 = 0; q0 < cnt; q0 += 256 * 16) {
        int cc[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int q = q0 + tid + 256 * u;
          cc[u] = q < cnt ? (codes ? codes[q] : q) : -1;
          if ((unsigned)cc[u] >= (unsigned)a.C) cc[u] = -1;
        }
        float lp[16], tg[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          lp[u] = cc[u] >= 0 ? (X ? lprow[cc[u]] - lse : lprow[cc[u]]) : -INFINITY;
          tg[u] = (G && cc[u] >= 0) ? noise_term(a, grow, cc[u], fl) : 0.0f;
        }
        // the best key of the round in the float domain, then the composite of its first
        // (lowest-code) position: the same maximum as over the composites
        float mk = -INFINITY;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float k = cc[u] >= 0 ? order_key<G>(s + lp[u], tg[u]) : -INFINITY;
          mk = k > mk ? k : mk;          // NaN keys never win
        }
        if (mk != -INFINITY) {
          int uf = 0;
#pragma unroll
          for (int u = 15; u >= 0; --u)
            if (cc[u] >= 0 && order_key<G>(s + lp[u], tg[u]) == mk) uf = u;
          best = max(best, candidate<G>(s, lp[uf], tg[uf], flat_base + (uint32_t)cc[uf], fl));
        }
      }
    }
  }
  if (pilot_contribute<G, WIDE>(a, pd, rd, best, S)) pilot_bound<G, PUBLISH, WIDE>(a, r, gsz, rd, S);
}

// The general kernels' pilots (the register-resident path runs its pilots inside
// select_pilot_beam_kernel).
template <bool G, bool X>
__global__ __launch_bounds__(256) void select_pilot_kernel(SelArgs a) {
  __shared__ PilotLds S;
  pilot_run<G, X, false, -1, true>(a, blockIdx.x, S);
}

// --------------------------------------------------------------------------------------
// per-beam top-k
// --------------------------------------------------------------------------------------
// Rows of any length (used when C > kOnePass): rows of up to kOnePass candidates in
// registers as above; longer rows stream through the LDS buffer.
template <bool G, bool X>
__global__ __launch_bounds__(256) void select_topk_kernel(SelArgs a) {
  __shared__ uint64_t buf[kSelCap];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scr[4];
  __shared__ uint64_t red64[8];
  __shared__ int red[4];
  __shared__ int cnt_s;
  const int tid = threadIdx.x;
  const int slot = blockIdx.x;
  const int r = a.slot_req[slot];
  const ReqDesc rd = a.req[r];
  const int j = slot - rd.boff;
  const float s = a.scores[slot];
  int fl = 0;
  int cnt = 0;
  const int32_t* codes = nullptr;
  uint32_t tau = a.bound[r];
  // a beam below the bound keeps nothing: no key exceeds its beam's score (noise can lift
  // an ordering key above the score, so the sampled selection reads every live beam)
  bool live = s != -INFINITY && !__builtin_isnan(s) && expands(a, slot, rd) && (G || ordered_key(s) >= tau);
  if (__builtin_isnan(s)) fl |= GRW_FLAG_NAN_LOGPROB;
  if (live && !beam_row(a, slot, cnt, codes)) {
    fl |= GRW_FLAG_BAD_NODE;
    live = false;
  }
  const float* lprow = a.logprobs + (size_t)slot * a.C;
  const float* grow = G ? a.noise + (size_t)slot * a.C : nullptr;
  const uint32_t flat_base = (uint32_t)j * (uint32_t)a.C;
  const int K = keep_k(a, rd);
  uint64_t* region = a.pool + rd.pool_off + (size_t)j * K;
  int n_out = 0;

  if (live && cnt <= kOnePass) {
    // ---- one pass: the row in registers, filtered by the bound, top K kept ----
    uint64_t v[kRegC];
    {
      RowRegs<kTrie, G> rr;  // row positions t + 256 k, codes kept (also for the full range)
      if (codes != nullptr) {
        load_row<kTrie, G>(rr, a, lprow, grow, codes, cnt, fl);
        if constexpr (X) {
          const float lse = a.row_lse[slot];
#pragma unroll
          for (int k = 0; k < kRegC; ++k) rr.lp[k] = rr.lp[k] - lse;
        }
      } else {
#pragma unroll
        for (int k = 0; k < kRegC; ++k) {
          const int i = tid + 256 * k;
          rr.code[k] = i < cnt ? i : -1;
          rr.lp[k] = i < cnt ? (X ? lprow[i] - a.row_lse[slot] : lprow[i]) : 0.0f;
          if constexpr (G) rr.tg[k] = i < cnt ? noise_term(a, grow, i, fl) : 0.0f;
        }
      }
#pragma unroll
      for (int k = 0; k < kRegC; ++k) {
        const uint32_t o = row_key<kTrie>(rr, k, cnt, s, 0u, fl);
        v[k] = o ? composite_key(o, flat_base + (uint32_t)rr.code[k]) : 0ull;
      }
    }
    int na = 0;
#pragma unroll
    for (int k = 0; k < kRegC; ++k) {
      if ((uint32_t)(v[k] >> 32) < tau) v[k] = 0;
      na += v[k] != 0;
    }
    const int n = block_sum256(na, red);
    if (n > 0) {
      uint64_t T = 1;
      n_out = n;
      if (n > K) {
        T = regs_select_threshold<256, kRegC>([&](int k) { return v[k]; }, K, hist, scr, red64);
        n_out = K;
      }
      if (n_out >= rd.W) {                       // this beam alone bounds the request's W-th best
        const uint64_t TW = (n_out == rd.W) ? T : regs_select_threshold<256, kRegC>([&](int k) { return v[k]; }, rd.W, hist, scr, red64);
        if (tid == 0) atomicMax(&a.bound[r], (uint32_t)(TW >> 32));
      }
      int ns = 0;
#pragma unroll
      for (int k = 0; k < kRegC; ++k) ns += (v[k] != 0 && v[k] >= T);
      int total;
      int p = block_excl_scan256(ns, red, &total);
#pragma unroll
      for (int k = 0; k < kRegC; ++k)
        if (v[k] != 0 && v[k] >= T) region[p++] = v[k];
      n_out = min(total, K);                     // the entries written (n_out by construction)
    }
  } else if (live && K >= cnt) {
    // ---- long row whose every candidate fits the region (a wide fan-out): no top-K, the
    // candidates at or above the bound go straight to the region ----
    if (tid == 0) cnt_s = 0;
    __syncthreads();
    for (int base = 0; base < cnt; base += 1024) {
      uint64_t e[4];
      int ne = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = base + tid + 256 * k;
        if (i < cnt) {
          const int c = codes ? codes[i] : i;
          if ((unsigned)c >= (unsigned)a.C) {
            fl |= GRW_FLAG_BAD_NODE;
            continue;
          }
          const float tg = G ? noise_term(a, grow, c, fl) : 0.0f;
          const float lp = X ? lprow[c] - a.row_lse[slot] : lprow[c];
          const uint64_t x = candidate<G>(s, lp, tg, flat_base + (uint32_t)c, fl);
          if (x != 0 && (uint32_t)(x >> 32) >= tau) e[ne++] = x;
        }
      }
      block_append<4>(region, &cnt_s, e, ne);
    }
    __syncthreads();
    n_out = cnt_s;
  } else if (live) {
    // ---- long rows: stream through the LDS buffer ----
    if (tid == 0) cnt_s = 0;
    __syncthreads();
    // rounds of kLongChunk candidates (8 per thread, their loads issued together, and the
    // next round's issued before this round is filtered); the buffer is trimmed to top K
    // (<= kSelCap - kLongChunk) before a round could overflow it
    constexpr int kLongChunk = 2048;
    static_assert(kMaxK + kLongChunk <= kSelCap, "a trimmed buffer must take a whole round");
    const float lse = X ? a.row_lse[slot] : 0.0f;
    auto load_round = [&](int base, int (&cc)[8], float (&lp)[8], float (&tg)[8]) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = base + tid + 256 * k;
        cc[k] = i < cnt ? (codes ? codes[i] : i) : -1;
        if (i < cnt && (unsigned)cc[k] >= (unsigned)a.C) {   // corrupt trie row: never read outside it
          fl |= GRW_FLAG_BAD_NODE;
          cc[k] = -1;
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        lp[k] = cc[k] >= 0 ? (X ? lprow[cc[k]] - lse : lprow[cc[k]]) : -INFINITY;
        tg[k] = (G && cc[k] >= 0) ? noise_term(a, grow, cc[k], fl) : 0.0f;
      }
    };
    // one round: trim if needed, filter the loaded candidates, append the survivors (reached
    // by every thread; two register sets alternate so that no loaded register is copied)
    int n = 0;
    auto run_round = [&](const int (&cc)[8], const float (&lp)[8], const float (&tg)[8]) __attribute__((always_inline)) {
      if (n + kLongChunk > kSelCap) {            // buffer full: keep the top K, raise tau
        const uint64_t T = block_select_threshold<256>([&](int i) { return buf[i]; }, n, K, hist, scr);
        n = block_compact_ge(buf, n, T, &cnt_s);
        const uint32_t tk = (uint32_t)(T >> 32);
        tau = max(tau, tk);
        tau = max(tau, __hip_atomic_load(&a.bound[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      }
      // admission in the float domain (key >= tau_f exactly when its ordered key >= tau, for
      // non-NaN keys); composites only for the admitted
      const float tau_f = tau < 0x00800000u ? -3.402823466e+38f : float_of_ordered(tau);
      uint64_t e[8];
      int ne = 0;
      bool suspect = false;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        suspect |= cc[k] >= 0 && !(lp[k] <= 0.0f);
        if (cc[k] >= 0 && order_key<G>(s + lp[k], tg[k]) >= tau_f) {
          const uint64_t x = candidate<G>(s, lp[k], tg[k], flat_base + (uint32_t)cc[k], fl);
          if (x != 0 && (uint32_t)(x >> 32) >= tau) e[ne++] = x;
        }
      }
      if (suspect) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (cc[k] < 0) continue;
          if (__builtin_isnan(lp[k])) fl |= GRW_FLAG_NAN_LOGPROB;
          else if (lp[k] > 0.0f) fl |= GRW_FLAG_POS_LOGPROB;
        }
      }
      block_append<8>(buf, &cnt_s, e, ne);
      lds_barrier();
      n = cnt_s;
    };
    int c0[8], c1[8];
    float l0[8], l1[8], t0[8], t1[8];
    load_round(0, c0, l0, t0);
    for (int base = 0; base < cnt; base += 2 * kLongChunk) {
      if (base + kLongChunk < cnt) load_round(base + kLongChunk, c1, l1, t1);
      run_round(c0, l0, t0);
      if (base + kLongChunk >= cnt) break;
      if (base + 2 * kLongChunk < cnt) load_round(base + 2 * kLongChunk, c0, l0, t0);
      run_round(c1, l1, t1);
    }
    uint64_t T = 1;
    n_out = n;
    if (n > K) {
      T = block_select_threshold<256>([&](int i) { return buf[i]; }, n, K, hist, scr);
      n_out = K;
    }
    if (n_out > 0) {
      if (n_out >= rd.W) {
        const uint64_t TW = (n_out == rd.W && n > K)
            ? T : block_select_threshold<256>([&](int i) { return buf[i]; }, n, rd.W, hist, scr);
        if (tid == 0) atomicMax(&a.bound[r], (uint32_t)(TW >> 32));
      }
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
        block_append<4>(region, &cnt_s, e, ne);
      }
      __syncthreads();
      n_out = min(cnt_s, K);                     // the entries written (n_out by construction)
    }
  }
  if (tid == 0) a.surv_count[slot] = n_out;
  fl = wave_butterfly(fl, [](int x, int y) { return x | y; });
  if ((tid & 63) == 0 && fl) atomicOr(a.flags, fl);
}

// --------------------------------------------------------------------------------------
// global W-of-pool select
// --------------------------------------------------------------------------------------
// Output slot `rank` of the request: token, parent, exact score, trie child.
// edge: the CSR edge of the entry when the per-beam stage recorded it (its child is node
// edge + 1), else -1 (the child is then found by a binary search of the parent's row).
// Without noise the entry's key is its score, fl32(score + lp), so the score is read from
// the composite; a zero key is recomputed from its operands, since the ordered key does not
// tell -0.0 from +0.0.  With noise (G) the key holds the noise and the score is recomputed.
template <bool G, bool X>
__device__ __forceinline__ void emit(const SelArgs& a, const ReqDesc& rd, int rank, uint64_t v, int edge = -1) {
  const int C = a.C;
  const int slot = rd.boff + rank;
  const uint32_t flat = composite_flat(v);
  const uint32_t b = flat / (uint32_t)C;
  const int c = (int)(flat - b * (uint32_t)C);
  if (b >= (uint32_t)rd.W) {                     // never for entries the per-beam stage wrote
    atomicOr(a.flags, (int)GRW_FLAG_POOL_CORRUPT);
    a.out_token[slot] = -1;
    a.out_parent[slot] = -1;
    a.out_score[slot] = -INFINITY;
    a.out_node[slot] = -1;
    return;
  }
  const int ps = rd.boff + (int)b;
  float score = G ? 0.0f : float_of_ordered((uint32_t)(v >> 32));
  if (G || score == 0.0f) {
    const float x = a.logprobs[(size_t)ps * C + c];
    score = a.scores[ps] + (X ? x - a.row_lse[ps] : x);
  }
  int node = -1;
  if (a.row_ptr != nullptr && edge >= 0) {
    node = edge + 1;
  } else if (a.row_ptr != nullptr) {
    const int pn = a.nodes[ps];
    int lo = a.row_ptr[pn], hi = a.row_ptr[pn + 1] - 1;
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
}

// Histogram bin of an entry: its key's distance below the origin in the float domain,
// times the bin scale, clamped to the NB bins.  Rounded float subtraction and
// multiplication are monotone, so the bin is non-increasing in the entry and the bins order
// the entries (ties inside a bin are ranked by full comparison).  The float domain keeps the
// bins even when the keys straddle zero, where ordered keys jump by about 2^31.
template <int NB>
__device__ __forceinline__ int hist_bin(uint64_t v, float origin, float scale) {
  const float d = (origin - float_of_ordered((uint32_t)(v >> 32))) * scale;
  return d < (float)(NB - 1) ? (d > 0.0f ? (int)d : 0) : NB - 1;
}

// beam of entry index i: the last b with pre[b] <= i (pre[0] = 0, pre[W] = n > i)
__device__ __forceinline__ int entry_beam(const uint32_t* pre, int W, uint32_t i) {
  int lo = 0, hi = W - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// LDS of the W-of-pool select: beam prefix (MAXW + 1), bin counts / cursors (NB), bin
// starts (NB + 1), winner array (WINCAP), radix histogram and small scratch.
template <int NT, int NB, int MAXW, int WINCAP, int EDGECAP = 1>
struct FinalLds {
  uint32_t pre[MAXW + 1];
  uint32_t hcnt[NB];
  uint32_t start[NB + 1];
  uint64_t win[WINCAP];
  int32_t wedge[EDGECAP];    // CSR edge of each placed entry (when EDGECAP == WINCAP)
  uint32_t hist[256];
  uint32_t scr[4];
  uint32_t wsum[NT / 64];
  uint32_t wmax[NT / 64];
  uint32_t tb, maxc;
  int cnt;
};

// The W_r-of-pool select of request r by one workgroup of NT threads (W_r <= MAXW).  The
// beams' survivor counts place every pool entry in one index range; a histogram of the
// entries' keys (bins measured down from the best live score, scaled so that the bound
// falls inside the range) finds the bin of the W_r-th best entry; the entries of that bin
// and of all better bins are placed bin by bin and ranked inside their bin, which gives
// every winner its output position.  When a bin holds more than BINCAP entries, a radix
// select and a bitonic sort in LDS do the same job.  Pool entries and counts are read with
// device-coherent loads (they may come from other workgroups of the same kernel).
// Survivor counts of request r's beams tid * BPT + k (device-coherent loads: the per-beam
// stage and the overflow rows write them), the thread's best live beam score as an ordered
// key (0 if none) and the request's bound, all in one round of loads.
struct FinalIn {
  uint32_t smax, bound;
};

template <int NT, int MAXW>
__device__ __forceinline__ FinalIn final_counts(const SelArgs& a, int r, const ReqDesc& rd, int32_t (&cnt)[MAXW / NT]) {
  const uint32_t bound = ld_dev(&a.bound[r]);
  uint32_t smax = 0;
#pragma unroll
  for (int k = 0; k < MAXW / NT; ++k) {
    const int b = (int)threadIdx.x * (MAXW / NT) + k;
    cnt[k] = b < rd.W ? ld_dev(&a.surv_count[rd.boff + b]) : 0;
    if (b < rd.W) {
      const float sc = a.scores[rd.boff + b];
      if (sc != -INFINITY && !__builtin_isnan(sc)) smax = max(smax, ordered_key(sc));
    }
  }
  return FinalIn{smax, bound};
}

template <int NT, int NB, int MAXW, int WINCAP, int BINCAP, int EDGECAP, bool G = false, bool X = false>
__device__ __forceinline__ void final_select(const SelArgs& a, int r, const ReqDesc& rd,
                                             FinalLds<NT, NB, MAXW, WINCAP, EDGECAP>& L, const int32_t (&cnt)[MAXW / NT],
                                             const FinalIn in) {
  constexpr bool EDGES = EDGECAP == WINCAP;   // entries carry their CSR edge (trie rows)
  constexpr int BPT = MAXW / NT;     // beams per thread
  constexpr int HPT = NB / NT;       // bins per thread
  constexpr int NRG = 8;             // pool entries cached per thread (and per batch beyond)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = rd.W, K = keep_k(a, rd);
  const uint64_t* pool = a.pool + rd.pool_off;
  uint32_t smax = in.smax;

  // beam prefix of the survivor counts, best live score
  uint32_t cb[BPT];
  uint32_t csum = 0;
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    cb[k] = min((uint32_t)cnt[k], (uint32_t)K);
    csum += cb[k];
  }
  {
    const uint32_t incl = (uint32_t)wave_inclusive_scan((int)csum);
    const uint32_t m = wave_max(smax);
    __syncthreads();
    if (lane == 63) L.wsum[wave] = incl;
    if (lane == 0) L.wmax[wave] = m;
    if (tid == 0) { L.tb = NB; L.maxc = 0; }
    __syncthreads();
    uint32_t run = incl - csum;
    for (int w = 0; w < wave; ++w) run += L.wsum[w];
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int b = tid * BPT + k;
      if (b < W) L.pre[b] = run;
      run += cb[k];
      if (b == W - 1) L.pre[W] = run;
    }
    smax = 0;
    for (int w = 0; w < NT / 64; ++w) smax = max(smax, L.wmax[w]);
  }
#pragma unroll
  for (int k = 0; k < HPT; ++k) L.hcnt[tid * HPT + k] = 0u;
  __syncthreads();
  const uint32_t n = L.pre[W];
  const int nsel = min((int)n, W);

  auto entry = [&](uint32_t i) {
    const int b = entry_beam(L.pre, W, i);
    return ld_dev(&pool[(size_t)b * K + (i - L.pre[b])]);
  };
  const bool edges = EDGES && a.row_ptr != nullptr;
  const int32_t* pedge = a.pool_edge + rd.pool_off;
  auto entry_edge = [&](uint32_t i) -> int {
    const int b = entry_beam(L.pre, W, i);
    return ld_dev(&pedge[(size_t)b * K + (i - L.pre[b])]);
  };
  const bool cached = n <= (uint32_t)(NT * NRG);
  uint64_t ev[NRG];
  int eg[NRG];
#pragma unroll
  for (int k = 0; k < NRG; ++k) {
    const uint32_t i = tid + NT * k;
    ev[k] = (cached && i < n) ? entry(i) : 0;
    eg[k] = (edges && cached && i < n) ? entry_edge(i) : -1;
  }
  // entries beyond the register cache are read in batches of NRG per thread
  auto for_each_entry = [&](auto&& fn) {
    if (cached) {
#pragma unroll
      for (int k = 0; k < NRG; ++k)
        if (ev[k]) fn(ev[k], eg[k]);
    } else {
      for (uint32_t base = 0; base < n; base += NT * NRG) {
        uint64_t bv[NRG];
        int be[NRG];
#pragma unroll
        for (int k = 0; k < NRG; ++k) {
          const uint32_t i = base + tid + NT * k;
          bv[k] = i < n ? entry(i) : 0;
          be[k] = (edges && i < n) ? entry_edge(i) : -1;
        }
#pragma unroll
        for (int k = 0; k < NRG; ++k)
          if (bv[k]) fn(bv[k], be[k]);
      }
    }
  };
  if constexpr (G) {
    // noise can lift an ordering key above every beam score: the bins start at the best entry
    uint32_t m = 0;
    for_each_entry([&](uint64_t v, int) { m = max(m, (uint32_t)(v >> 32)); });
    m = wave_max(m);
    __syncthreads();
    if (lane == 0) L.wmax[wave] = m;
    __syncthreads();
    smax = 0;
    for (int w = 0; w < NT / 64; ++w) smax = max(smax, L.wmax[w]);
  }

  // histogram origin and scale: bins reach from the best live score (the best entry with
  // noise) down to the bound
  uint32_t lo = in.bound;
  if (lo == 0 && smax != 0) {
    const uint32_t u = (smax & 0x80000000u) ? (smax & 0x7fffffffu) : ~smax;   // inverse ordered key
    lo = ordered_key(__uint_as_float(u) - 64.0f);
  }
  const float org = float_of_ordered(smax), lo_f = float_of_ordered(lo);
  const float width = org - lo_f;      // >= 0; bins of width / (NB - 1)
  const float scale = width > 0.0f && width < 3.0e38f ? (float)(NB - 1) / width : 0.0f;

  for_each_entry([&](uint64_t v, int) { atomicAdd(&L.hcnt[hist_bin<NB>(v, org, scale)], 1u); });
  __syncthreads();

  // bin starts: exclusive scan of the histogram; the bin tb of the nsel-th entry and, from a
  // prefix maximum taken in the same pass, the largest count among bins <= tb
  {
    uint32_t c[HPT];
    uint32_t tsum = 0, tmax = 0;
#pragma unroll
    for (int k = 0; k < HPT; ++k) { c[k] = L.hcnt[tid * HPT + k]; tsum += c[k]; tmax = max(tmax, c[k]); }
    const uint32_t incl = (uint32_t)wave_inclusive_scan((int)tsum);
    const uint32_t imax = wave_inclusive_max_scan(tmax);
    __syncthreads();
    if (lane == 63) { L.wsum[wave] = incl; L.wmax[wave] = imax; }
    __syncthreads();
    uint32_t run = incl - tsum;
    uint32_t pmax = lane_before(imax);   // maximum over the earlier lanes' bins
    for (int w = 0; w < wave; ++w) { run += L.wsum[w]; pmax = max(pmax, L.wmax[w]); }
#pragma unroll
    for (int k = 0; k < HPT; ++k) {
      pmax = max(pmax, c[k]);
      L.start[tid * HPT + k] = run;
      if (nsel > 0 && run < (uint32_t)nsel && (uint32_t)nsel <= run + c[k]) { L.tb = tid * HPT + k; L.maxc = pmax; }
      run += c[k];
    }
    if (tid == NT - 1) L.start[NB] = run;
  }
  __syncthreads();
  const uint32_t tb = L.tb;
  const bool fast = nsel > 0 && tb < (uint32_t)NB && L.maxc <= (uint32_t)BINCAP && L.start[tb + 1] <= (uint32_t)WINCAP;

  if (fast) {
    // place every entry of bins <= tb in its bin's segment (counting the bin's count down),
    // then rank it inside the bin
    auto place = [&](uint64_t v, int e) {
      const int b = hist_bin<NB>(v, org, scale);
      if ((uint32_t)b <= tb) {
        const uint32_t p = L.start[b] + atomicSub(&L.hcnt[b], 1u) - 1u;
        if (p < L.start[b + 1]) {
          L.win[p] = v;
          if constexpr (EDGES) L.wedge[p] = e;
        }
      }
    };
    for_each_entry(place);
    __syncthreads();
    const int m = (int)L.start[tb + 1];
    for (int p = tid; p < m; p += NT) {
      const uint64_t v = L.win[p];
      const int b = hist_bin<NB>(v, org, scale);
      const int s0 = (int)L.start[b], e0 = (int)L.start[b + 1];
      int rank = s0;
      for (int q = s0; q < e0; ++q) rank += L.win[q] > v;
      if (rank < nsel) emit<G, X>(a, rd, rank, v, EDGES ? L.wedge[p] : -1);
    }
  } else if (nsel > 0) {
    // fallback: radix select of the W-th entry, gather, bitonic sort
    uint64_t T = 0;
    if ((int)n > W) T = block_select_threshold<NT>([&](int i) { return entry((uint32_t)i); }, (int)n, W, L.hist, L.scr);
    if (tid == 0) L.cnt = 0;
    __syncthreads();
    for (uint32_t base = 0; base < n; base += NT) {
      const uint32_t i = base + tid;
      uint64_t e[1];
      int ne = 0;
      if (i < n) {
        const uint64_t v = entry(i);
        if (v >= T) e[ne++] = v;
      }
      block_append<1>(L.win, &L.cnt, e, ne);
    }
    __syncthreads();
    int npow = 1;
    while (npow < nsel) npow <<= 1;
    for (int i = nsel + tid; i < npow; i += NT) L.win[i] = 0ull;   // sorts last
    __syncthreads();
    for (int k = 2; k <= npow; k <<= 1) {
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        for (int i = tid; i < npow; i += NT) {
          const int ixj = i ^ jj;
          if (ixj > i) {
            const uint64_t x = L.win[i], y = L.win[ixj];
            const bool desc = (i & k) == 0;
            if (desc ? (x < y) : (x > y)) {
              L.win[i] = y;
              L.win[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < nsel; i += NT) emit<G, X>(a, rd, i, L.win[i]);
  }
  for (int i = nsel + tid; i < W; i += NT) {
    const int slot = rd.boff + i;
    a.out_token[slot] = -1;
    a.out_parent[slot] = -1;
    a.out_score[slot] = -INFINITY;
    a.out_node[slot] = -1;
  }
}

constexpr int kGlobThreads = 1024;
constexpr int kGlobWinCap = kMaxW + kBinCap;
typedef FinalLds<kGlobThreads, kHistBins, kMaxW, kGlobWinCap, 1> GlobLds;

template <bool G, bool X>
__global__ __launch_bounds__(kGlobThreads) void select_global_kernel(SelArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  GlobLds& L = *(GlobLds*)smem;
  int32_t cnt[kMaxW / kGlobThreads];
  const ReqDesc rd = a.req[blockIdx.x];
  const FinalIn in = final_counts<kGlobThreads, kMaxW>(a, blockIdx.x, rd, cnt);
  final_select<kGlobThreads, kHistBins, kMaxW, kGlobWinCap, kBinCap, 1, G, X>(a, blockIdx.x, rd, L, cnt, in);
  if (threadIdx.x == 0) a.bound[blockIdx.x] = 0u;
}

// --------------------------------------------------------------------------------------
// register-resident step: per-beam stage, then the W-of-pool stage
// --------------------------------------------------------------------------------------
// Used when every row fits the one-read path (C <= kOnePass) and W <= kFusedMaxW.  The
// pilot + per-beam kernel runs one small workgroup per pilot and per beam slot (no large
// LDS arrays); the W-of-pool kernel runs one 1024-thread workgroup per request.
constexpr int kFusedMaxW = 1024;
constexpr int kFusedBins = 1024;
constexpr int kFusedBinCap = 512;
constexpr int kFusedWinCap = kFusedMaxW + kFusedBinCap;

struct BeamRow {
  int slot, r, cnt;
  int beg;             // first CSR edge of the beam's trie row
  float s;
  bool live;
  uint32_t tau;        // the request's bound
  ReqDesc rd;
  const int32_t* codes;
  const uint32_t* mask;  // dense child mask of the node, or NULL (CSR row)
  const float* lprow;
};

// read_bound: false when the bound is published during the same kernel (the caller then
// waits for it and sets b.tau; no plain load may cache the word before that)
__device__ __forceinline__ BeamRow beam_setup(const SelArgs& a, int slot, int& fl, bool read_bound = true) {
  BeamRow b;
  b.slot = slot;
  b.r = a.slot_req[slot];
  b.s = a.scores[slot];
  b.rd = a.req[b.r];           // descriptor and bound are read before the row
  b.tau = read_bound ? a.bound[b.r] : 0u;
  b.cnt = a.C;
  b.codes = nullptr;
  b.mask = nullptr;
  b.lprow = a.logprobs + (size_t)slot * a.C;
  b.beg = 0;
  b.live = b.s != -INFINITY && !__builtin_isnan(b.s) && expands(a, slot, b.rd);
  if (__builtin_isnan(b.s)) fl |= GRW_FLAG_NAN_LOGPROB;
  if (b.live && !beam_row(a, slot, b.cnt, b.codes, &b.mask)) {
    fl |= GRW_FLAG_BAD_NODE;
    b.live = false;
  }
  if (b.live && b.codes != nullptr) b.beg = (int)(b.codes - a.code);
  if (b.live && b.cnt > kOnePass) {              // longer than the code range: corrupt row
    fl |= GRW_FLAG_BAD_NODE;
    b.live = false;
  }
  return b;
}

// Survivors of one loaded beam row: candidates >= the request's bound, stored in the beam's
// pool region.  Returns the survivor count.  When the row has more than top_k of them:
// without noise (rare once the bound is set) it returns -1 and stores nothing, and the
// request's W-of-pool workgroup selects that row's top_k; with noise (G), where it happens
// to several beams per step, a radix select over the registers keeps the top_k here.
// Reached by every thread of the workgroup.
// What a thread of a beam workgroup can learn from its loaded row before the bound is
// known: its largest ordering key (NaN keys ignored; -inf when it holds none) and whether
// any of its positions holds a NaN or positive log-probability.
struct RowPre {
  float best;
  bool suspect;
};
template <int L, bool G>
__device__ __forceinline__ RowPre row_pre(const BeamRow& b, const RowRegs<L, G>& rr) {
  RowPre p{-INFINITY, false};
  if constexpr (G) {
#pragma unroll
    for (int k = 0; k < kRegC; ++k) {
      p.suspect |= !(rr.lp[k] <= 0.0f);
      p.best = fmaxf(p.best, order_key<G>(b.s + rr.lp[k], rr.tg[k]));
    }
  } else {
    // rounded addition is monotonic: the largest s + lp is s + the largest lp
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kRegC; ++k) {
      p.suspect |= !(rr.lp[k] <= 0.0f);
      m = fmaxf(m, rr.lp[k]);
    }
    p.best = b.s + m;
  }
  return p;
}

template <int L, bool G>
__device__ __forceinline__ int keep_beam(const SelArgs& a, const BeamRow& b, const RowRegs<L, G>& rr, const RowPre& pre,
                                         int& fl, int* red, uint32_t* hist, uint32_t* scr, uint32_t* red32,
                                         uint32_t* mwords, uint32_t* mprefix) {
  const ReqDesc& rd = b.rd;
  const uint32_t tau = b.tau;
  // a beam below the bound keeps nothing: no key exceeds its beam's score (with noise an
  // ordering key can exceed it, so every live beam is read)
  if (!b.live || (!G && ordered_key(b.s) < tau)) return 0;
  const int j = b.slot - rd.boff;
  const uint32_t flat_base = (uint32_t)j * (uint32_t)a.C;
  // Admission in the float domain: for a non-NaN key, key >= tau_f exactly when its
  // ordered key is >= tau (-0.0 and +0.0 compare equal on both sides); NaN keys and the -inf
  // of positions without a candidate never pass.  Most rows admit a handful of candidates,
  // so ordered keys are formed only for those.
  const float tau_f = tau < 0x00800000u ? -3.402823466e+38f : float_of_ordered(tau);   // -FLT_MAX: every finite key
  // only a thread whose best key reaches the bound looks at its positions
  int na = 0;
  if (pre.best >= tau_f) {
#pragma unroll
    for (int k = 0; k < kRegC; ++k) na += order_key<G>(b.s + rr.lp[k], G ? rr.tg[k] : 0.0f) >= tau_f;
  }
  if (pre.suspect) {                             // NaN or positive: a precondition flag
#pragma unroll
    for (int k = 0; k < kRegC; ++k) {
      if (__builtin_isnan(rr.lp[k])) fl |= GRW_FLAG_NAN_LOGPROB;
      else if (rr.lp[k] > 0.0f) fl |= GRW_FLAG_POS_LOGPROB;
    }
  }
  int n;
  int p = block_excl_scan<256>(na, red, &n);
  if (n == 0) return 0;
  const int K = keep_k(a, rd);
  uint64_t* region = a.pool + rd.pool_off + (size_t)j * K;
  int32_t* redge = a.pool_edge + rd.pool_off + (size_t)j * K;
  // CSR edge of a survivor: position t + 256 k of a CSR row; in a dense row the rank of its
  // code among the node's children (popcount of the mask below it)
  if constexpr (L == kTrie) {
    if (b.mask != nullptr) {
      const int w = threadIdx.x;
      const uint32_t m = w < a.mask_words ? b.mask[w] : 0u;   // mask_words <= 256 on this path
      mwords[w] = m;
      int tot;
      mprefix[w] = (uint32_t)block_excl_scan<256>(__builtin_popcount(m), red, &tot);
      __syncthreads();
    }
  }
  auto edge_of = [&](int k) -> int {
    if constexpr (L == kTrie) {
      if (b.mask == nullptr) return b.beg + (int)threadIdx.x + 256 * k;
      const int c = rr.code[k];
      const int e = b.beg + (int)mprefix[c >> 5] + __builtin_popcount(mwords[c >> 5] & ((1u << (c & 31)) - 1u));
      // a mask bit must name a code of the CSR row: the rank is that code's edge.  Otherwise
      // the code is no child of the node; the W-of-pool stage's search then finds no child
      // either (node -1) and both flag it
      if (e >= b.beg + b.cnt || a.code[e] != c) {
        fl |= GRW_FLAG_CHILD_MISSING;
        return -1;
      }
      return e;
    } else {
      return -1;
    }
  };
  if (n > K) {
    if constexpr (!G) {
      return -1;
    } else {
      auto key = [&](int k) -> uint32_t {
        const float kf = order_key<G>(b.s + rr.lp[k], rr.tg[k]);
        return kf >= tau_f ? ordered_key(kf) : 0u;
      };
      auto flat = [&](int k) -> uint32_t { return flat_base + (uint32_t)rr.code_of(k); };
      const uint64_t T = regs_select_composite<256, kRegC>(key, flat, K, n, hist, scr, red32);
      const uint32_t thi = (uint32_t)(T >> 32), tlo = (uint32_t)T;
      uint32_t keep = 0;
#pragma unroll
      for (int k = 0; k < kRegC; ++k) {
        const uint32_t ok = key(k);
        if (ok > thi || (ok == thi && ok != 0u && ~flat(k) >= tlo)) keep |= 1u << k;
      }
      int total;
      int q = block_excl_scan<256>(__builtin_popcount(keep), red, &total);
#pragma unroll
      for (int k = 0; k < kRegC; ++k) {
        if ((keep >> k) & 1u) {
          if constexpr (L == kTrie) redge[q] = edge_of(k);
          region[q++] = composite_key(key(k), flat(k));
        }
      }
      return min(total, K);
    }
  }
#pragma unroll
  for (int k = 0; k < kRegC; ++k) {
    const float kf = order_key<G>(b.s + rr.lp[k], G ? rr.tg[k] : 0.0f);
    if (kf >= tau_f) {
      if constexpr (L == kTrie) redge[p] = edge_of(k);
      region[p++] = composite_key(ordered_key(kf), flat_base + (uint32_t)rr.code_of(k));
    }
  }
  return n;
}

// The top_k survivors of an overflowing beam row (more than top_k candidates >= the bound),
// by the NT threads of the request's W-of-pool workgroup: the row is read again, NR
// positions per thread (rows of at most NT * NR candidates), a radix select finds the
// top_k-th composite, and the survivors go to the beam's pool region.
template <int NT, int NR, bool G, bool X>
__device__ __forceinline__ void overflow_row(const SelArgs& a, const ReqDesc& rd, int r, int slot, uint32_t* hist,
                                             uint32_t* scr, uint32_t* red32, int* red) {
  const int tid = threadIdx.x;
  const int j = slot - rd.boff;
  const float s = a.scores[slot];
  int cnt = a.C;
  const int32_t* codes = nullptr;
  if (!beam_row(a, slot, cnt, codes) || cnt > NT * NR) {   // never for rows the beam stage admitted
    if (tid == 0) st_dev(&a.surv_count[slot], 0);
    return;
  }
  const uint32_t tau = ld_dev(&a.bound[r]);
  const float tau_f = tau < 0x00800000u ? -3.402823466e+38f : float_of_ordered(tau);
  const float* lprow = a.logprobs + (size_t)slot * a.C;
  const uint32_t flat_base = (uint32_t)j * (uint32_t)a.C;
  const int beg = codes != nullptr ? (int)(codes - a.code) : 0;
  const float* grow = G ? a.noise + (size_t)slot * a.C : nullptr;
  float lp[NR];
  float tg[G ? NR : 1];
  int code[NR];
  int na = 0, fl = 0;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int i = tid + NT * k;
    code[k] = i < cnt ? (codes != nullptr ? codes[i] : i) : -1;
    if ((unsigned)code[k] >= (unsigned)a.C) code[k] = -1;
    lp[k] = code[k] >= 0 ? lprow[code[k]] : -INFINITY;
    if constexpr (X) lp[k] = lp[k] - a.row_lse[slot];
    if constexpr (G) tg[k] = code[k] >= 0 ? noise_term(a, grow, code[k], fl) : 0.0f;
    na += order_key<G>(s + lp[k], G ? tg[k] : 0.0f) >= tau_f;
  }
  int n;
  (void)block_excl_scan<NT>(na, red, &n);
  const int K = keep_k(a, rd);
  auto key = [&](int k) -> uint32_t {
    const float kf = order_key<G>(s + lp[k], G ? tg[k] : 0.0f);
    return kf >= tau_f ? ordered_key(kf) : 0u;
  };
  auto flat = [&](int k) -> uint32_t { return flat_base + (uint32_t)code[k]; };
  const uint64_t T = n > K ? regs_select_composite<NT, NR>(key, flat, K, n, hist, scr, red32) : 1ull;
  const uint32_t thi = (uint32_t)(T >> 32), tlo = (uint32_t)T;
  uint32_t keep = 0;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const uint32_t ok = key(k);
    if (ok > thi || (ok == thi && ok != 0u && ~flat(k) >= tlo)) keep |= 1u << k;
  }
  int total;
  int p = block_excl_scan<NT>(__builtin_popcount(keep), red, &total);
  uint64_t* region = a.pool + rd.pool_off + (size_t)j * K;
  int32_t* redge = a.pool_edge + rd.pool_off + (size_t)j * K;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    if ((keep >> k) & 1u) {
      if (codes != nullptr) st_dev(&redge[p], beg + tid + NT * k);
      st_dev(&region[p++], composite_key(key(k), flat(k)));
    }
  }
  if (tid == 0) st_dev(&a.surv_count[slot], min(total, K));
}

// The per-beam stage with the pilots in the same launch.  Workgroups [0, n_pilots) are the
// pilots and never wait; every later workgroup takes one beam slot, issues its row loads,
// and then waits until its request's last pilot has published the bound.  Workgroups are
// dispatched in index order, so every pilot is resident or finished before a workgroup
// that waits for it starts, and the waiting workgroups' row loads overlap the pilots'
// work.  The wait is bounded: after a.wait_limit polls the workgroup proceeds with bound 0,
// which admits every candidate and leaves its row to the overflow path (slower, same
// result).
//
// Thread 0 polls its copy of request r's step word until `bit` is set (at most
// a.wait_limit polls); every thread gets the last value read.
__device__ __forceinline__ uint64_t wait_sync(const SelArgs& a, int r, uint64_t bit, uint64_t* word) {
  if (threadIdx.x == 0) {
    const uint64_t* p = &a.sync[((size_t)r * kSyncCopies + blockIdx.x % kSyncCopies) * kSyncStride];
    uint64_t v = 0;
    for (int i = 0; i < a.wait_limit; ++i) {
      v = ld_dev(p);
      if (v & bit) break;
      __builtin_amdgcn_s_sleep(2);
    }
    *word = v;
  }
  __syncthreads();
  const uint64_t v = *word;
  __syncthreads();
  return v;
}

// Waves per SIMD the pilot + per-beam kernel is built for: with plain full rows every beam
// workgroup's row fits in 64 registers per lane, so 8 workgroups per CU are resident.
template <int L, bool G, bool X>
constexpr int pilot_beam_waves() { return (L == kFull && !G && !X) ? 8 : 1; }

template <int L, bool G, bool X>
__global__ __launch_bounds__(256, (pilot_beam_waves<L, G, X>())) void select_pilot_beam_kernel(SelArgs a) {
  __shared__ PilotLds S;
  __shared__ uint32_t mwords[L == kTrie ? 256 : 1];
  __shared__ uint32_t mprefix[L == kTrie ? 256 : 1];
  __shared__ uint64_t word_s;
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < a.n_pilots) {
    pilot_run<G, X, true, L>(a, blockIdx.x, S);
    return;
  }
  const int slot = blockIdx.x - a.n_pilots;
  int fl = 0;
  RowRegs<L, G> rr;
  int lfl = 0;
  if constexpr (L != kTrie)    // full rows: loads before the descriptor loads, kept if the beam is live
    load_row<L, G>(rr, a, a.logprobs + (size_t)slot * a.C, G ? a.noise + (size_t)slot * a.C : nullptr, nullptr, a.C, lfl);
  BeamRow b = beam_setup(a, slot, fl, false);
  if constexpr (L == kTrie) {
    if (b.live) load_row<L, G>(rr, a, b.lprow, G ? a.noise + (size_t)slot * a.C : nullptr, b.codes, b.cnt, fl, b.mask);
  } else if (b.live) {
    fl |= lfl;
  }
  // every slot computes its own row lse (a pilot slot's equals its pilot's: same layout, same
  // reduction order)
  if constexpr (X)
    if (b.live) to_logprobs<L, G>(rr, a, slot, b.lprow, true, S.redf, S.redd, fl);
  // the work that does not need the bound is done while the pilots finish
  const RowPre pre = b.live ? row_pre<L, G>(b, rr) : RowPre{-INFINITY, false};
  // a dead or non-expanding slot keeps nothing and needs no bound (b.live is uniform)
  const uint64_t w = b.live ? wait_sync(a, b.r, kSyncBound, &word_s) : 0ull;
  b.tau = (w & kSyncBound) ? (uint32_t)w : 0u;
  const int n_out = keep_beam<L, G>(a, b, rr, pre, fl, S.red, S.hist, S.scr, S.red32, mwords, mprefix);
  if (tid == 0) a.surv_count[slot] = n_out;
  fl = wave_butterfly(fl, [](int x, int y) { return x | y; });
  if ((tid & 63) == 0 && fl) atomicOr(a.flags, fl);
}

// W-of-pool stage: one workgroup of 1024 threads per request, after every beam's survivors
// are in the pool; resets the request's bound for the next step.
constexpr int kFinThreads = 1024;
typedef FinalLds<kFinThreads, kFusedBins, kFusedMaxW, kFusedWinCap, kFusedWinCap> FinLds;

template <bool G, bool X>
__global__ __launch_bounds__(kFinThreads) void select_final_kernel(SelArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  FinLds& L = *(FinLds*)smem;
  __shared__ int red[kFinThreads / 64];
  __shared__ uint32_t red32[2 * (kFinThreads / 64)];
  __shared__ int n_over;
  const int r = blockIdx.x;
  const ReqDesc rd = a.req[r];
  constexpr int BPT = kFusedMaxW / kFinThreads;
  int32_t cnt[BPT];
  FinalIn in = final_counts<kFinThreads, kFusedMaxW>(a, r, rd, cnt);
  // beams whose rows overflowed top_k (negative counts): their survivors first (listed in
  // L.pre meanwhile); the counts are read again after them
  if (threadIdx.x == 0) n_over = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < BPT; ++k)
    if (cnt[k] < 0) L.pre[atomicAdd(&n_over, 1)] = (uint32_t)(rd.boff + (int)threadIdx.x * BPT + k);
  __syncthreads();
  const int no = n_over;
  if (no > 0) {
    for (int i = 0; i < no; ++i) {
      const int slot = (int)L.pre[i];
      __syncthreads();
      overflow_row<kFinThreads, kOnePass / kFinThreads, G, X>(a, rd, r, slot, L.hist, L.scr, red32, red);
    }
    wait_stores();
    __syncthreads();
    in = final_counts<kFinThreads, kFusedMaxW>(a, r, rd, cnt);
  }
  final_select<kFinThreads, kFusedBins, kFusedMaxW, kFusedWinCap, kFusedBinCap, kFusedWinCap, G, X>(a, r, rd, L, cnt, in);
  __syncthreads();
  if (threadIdx.x == 0) a.bound[r] = 0u;
  if (threadIdx.x < kSyncCopies) a.sync[((size_t)r * kSyncCopies + threadIdx.x) * kSyncStride] = 0ull;
}

// Row lse of every live beam slot for the general kernels (rows of any length, read with
// stride 256 twice: max, then the float64 sum of exp(x - max)).
__global__ __launch_bounds__(256) void select_lse_kernel(SelArgs a) {
  __shared__ float redf[4];
  __shared__ double redd[4];
  const int slot = blockIdx.x;
  const float s = a.scores[slot];
  if (s == -INFINITY || __builtin_isnan(s)) return;
  const float* xrow = a.logprobs + (size_t)slot * a.C;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int fl = 0;
  float m = -INFINITY;
  for (int i = threadIdx.x; i < a.C; i += 256) {
    const float x = xrow[i];
    if (__builtin_isnan(x) || x == INFINITY) fl |= GRW_FLAG_NAN_LOGPROB;
    m = fmaxf(m, x);
  }
  m = wave_max(m);
  if (lane == 0) redf[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(redf[0], redf[1]), fmaxf(redf[2], redf[3]));
  const double md = (double)m;
  double sum = 0.0;
  for (int i = threadIdx.x; i < a.C; i += 256) sum += exp((double)xrow[i] - md);
  sum = wave_sum(sum);
  if (lane == 0) redd[wave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) a.row_lse[slot] = (float)(md + log(((redd[0] + redd[1]) + redd[2]) + redd[3]));
  fl = wave_butterfly(fl, [](int x, int y) { return x | y; });
  if (lane == 0 && fl) atomicOr(a.flags, fl);
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

template <bool G, bool X>
hipError_t select_topk_path(const SelArgs& a, hipStream_t s) {
  if (X) select_lse_kernel<<<a.sumW, 256, 0, s>>>(a);
  select_pilot_kernel<G, X><<<a.n_pilots, 256, 0, s>>>(a);
  select_topk_kernel<G, X><<<a.sumW, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_select_topk(const SelArgs& a, hipStream_t s) {
  if (a.sumW == 0) return hipSuccess;
  const bool g = a.noise != nullptr, x = a.row_lse != nullptr;
  if (g) return x ? select_topk_path<true, true>(a, s) : select_topk_path<true, false>(a, s);
  return x ? select_topk_path<false, true>(a, s) : select_topk_path<false, false>(a, s);
}

template <bool G, bool X>
hipError_t select_global_path(const SelArgs& a, hipStream_t s) {
  static bool attr_set = false;   // the bin arrays and winner array exceed the default 64 KB
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)select_global_kernel<G, X>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(GlobLds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  select_global_kernel<G, X><<<a.R, kGlobThreads, sizeof(GlobLds), s>>>(a);
  return hipGetLastError();
}

hipError_t launch_select_global(const SelArgs& a, hipStream_t s) {
  if (a.R == 0) return hipSuccess;
  const bool g = a.noise != nullptr, x = a.row_lse != nullptr;
  if (g) return x ? select_global_path<true, true>(a, s) : select_global_path<true, false>(a, s);
  return x ? select_global_path<false, true>(a, s) : select_global_path<false, false>(a, s);
}

bool select_fused_ok(int C, int max_W) { return C <= kOnePass && max_W <= kFusedMaxW; }

template <bool G, bool X>
hipError_t select_fused_path(const SelArgs& a, hipStream_t s) {
  static bool attr_set = false;   // the W-of-pool select's arrays exceed the default 64 KB
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)select_final_kernel<G, X>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(FinLds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = a.n_pilots + a.sumW;     // pilots first, then one workgroup per slot
  const bool aligned = (((uintptr_t)a.logprobs) & 15) == 0 && (!G || (((uintptr_t)a.noise) & 15) == 0);
  if (a.row_ptr != nullptr)
    select_pilot_beam_kernel<kTrie, G, X><<<grid, 256, 0, s>>>(a);
  else if ((a.C & 3) == 0 && aligned)
    select_pilot_beam_kernel<kFull, G, X><<<grid, 256, 0, s>>>(a);
  else
    select_pilot_beam_kernel<kFullScalar, G, X><<<grid, 256, 0, s>>>(a);
  select_final_kernel<G, X><<<a.R, kFinThreads, sizeof(FinLds), s>>>(a);
  return hipGetLastError();
}

hipError_t launch_select_fused(const SelArgs& a, hipStream_t s) {
  if (a.sumW == 0) return hipSuccess;
  const bool g = a.noise != nullptr, x = a.row_lse != nullptr;
  if (g) return x ? select_fused_path<true, true>(a, s) : select_fused_path<true, false>(a, s);
  return x ? select_fused_path<false, true>(a, s) : select_fused_path<false, false>(a, s);
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
