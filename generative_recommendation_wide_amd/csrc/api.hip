// C-ABI layer: workspace, argument validation, batch binding and kernel dispatch.
//
// Everything the decode step needs on the device is allocated once in grw_ws_create
// (xLLM generative-recommendation design doc, section 3.2: prepare the space, indices and
// structures of later steps up front; section 4.3: reuse candidate containers instead of
// creating them every round).  grw_ws_bind_batch uploads per-request descriptors and the
// shared-stage work list once per batch; the per-step calls only enqueue kernels.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <numeric>
#include <vector>

#include "grw_internal.h"

using namespace grw;

struct grw_ws {
  grw_limits lim;
  int device = 0;
  int n_cu = 256;
  bool mfma = false;            // shared stage on the bf16 MFMA kernel
  // device buffers
  ReqDesc* d_req = nullptr;
  int32_t* d_slot_req = nullptr;
  ShWork* d_work = nullptr;
  int64_t work_cap = 0;
  float* d_opart = nullptr;
  float* d_lpart = nullptr;
  float* d_ou = nullptr;
  float* d_lu = nullptr;
  uint64_t* d_pool = nullptr;
  int32_t* d_pool_edge = nullptr;
  int64_t pool_cap = 0;
  int32_t* d_surv_count = nullptr;
  uint32_t* d_bound = nullptr;
  int32_t* d_pilot_desc = nullptr;
  float* d_row_lse = nullptr;       // [max_total_beams] row lse of the selection from raw logits
  uint64_t* d_pilot_buf = nullptr;
  uint32_t* d_step_state = nullptr;    // [max_requests]: pilots finished in the current step
  uint64_t* d_sync = nullptr;          // [max_requests][kSyncCopies * kSyncStride] step-state words
  int32_t* d_flags = nullptr;
  // fork and join events of the two-stream attention
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // pinned host staging for the bind upload
  void* h_stage = nullptr;
  size_t stage_bytes = 0;
  // bound batch (host mirror)
  bool bound = false;
  int R = 0;
  int sumW = 0;
  int maxW = 0, maxK = 0;
  int n_work = 0;
  int n_wide = 0;                // leading items of the work list that use the 8-wave kernel
  int n_pilots = 0;              // pilot workgroups of the deterministic selection
  int n_pilots_s = 0;            // pilot workgroups of the sampled selection
  int n_pilots_w = 0;            // ... of the general kernels, deterministic
  int n_pilots_ws = 0;           // ... of the general kernels, sampled
  int pilot_cap = 0;             // pilot-buffer entries per request
  int32_t wait_limit = kBoundSpin;   // polls of a beam workgroup waiting for its bound
  std::vector<ReqDesc> req;
};

namespace {

int hip_status(hipError_t e) { return e == hipSuccess ? GRW_OK : GRW_EDEVICE; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool dtype_ok(int t) { return t == GRW_F32 || t == GRW_BF16 || t == GRW_FP8_E4M3; }

int64_t mfma_items_bound(const grw_limits& L, int g) {
  const int64_t mt = ceil_div((int64_t)L.max_total_beams * g, kShRows) + L.max_requests;
  return (int64_t)L.Hkv * mt * L.max_splits;
}

template <typename T>
int dev_alloc(T** p, int64_t n) {
  if (n <= 0) n = 1;
  if (hipMalloc((void**)p, (size_t)n * sizeof(T)) != hipSuccess) {
    *p = nullptr;
    return GRW_ENOMEM;
  }
  return GRW_OK;
}

void free_all(grw_ws* w) {
  (void)hipFree(w->d_req);
  (void)hipFree(w->d_slot_req);
  (void)hipFree(w->d_work);
  (void)hipFree(w->d_opart);
  (void)hipFree(w->d_lpart);
  (void)hipFree(w->d_ou);
  (void)hipFree(w->d_lu);
  (void)hipFree(w->d_pool);
  (void)hipFree(w->d_pool_edge);
  (void)hipFree(w->d_surv_count);
  (void)hipFree(w->d_bound);
  (void)hipFree(w->d_pilot_desc);
  (void)hipFree(w->d_row_lse);
  (void)hipFree(w->d_step_state);
  (void)hipFree(w->d_sync);
  (void)hipFree(w->d_pilot_buf);
  (void)hipFree(w->d_flags);
  if (w->h_stage) (void)hipHostFree(w->h_stage);
  if (w->ev_fork) (void)hipEventDestroy(w->ev_fork);
  if (w->ev_join) (void)hipEventDestroy(w->ev_join);
}

// Shared-stage work lists of the MFMA kernels.  Requests with bf16 KV and more than 128
// query rows per kv head go to the 8-wave kernel (256 rows per item); the others to the
// 4-wave kernel (128 rows).  Items of one (request, kv head, split) share the same prompt
// tiles; they are assigned to one XCD (workgroup i runs on XCD i % 8) so the repeated tile
// reads are served by that XCD's L2.  The wide list comes first, then the narrow one.
void build_mfma_work(grw_ws* w, std::vector<ShWork>& out, int& n_wide) {
  const grw_limits& L = w->lim;
  const int g = L.Hq / L.Hkv;
  auto is_wide = [&](const ReqDesc& r) {
    return L.kv_dtype == GRW_BF16 && (int64_t)r.W * g > kShRows;
  };
  // balance: aim for about two 4-wave workgroups' worth of work per CU (a wide item counts
  // twice), splitting long prompts
  int64_t total_units = 0;
  for (const ReqDesc& r : w->req) {
    const int rows = is_wide(r) ? kShRowsWide : kShRows;
    total_units += (int64_t)L.Hkv * ceil_div((int64_t)r.W * g, rows) * (rows / kShRows) * ceil_div(r.P, kShKeys);
  }
  const int64_t target_units = 2LL * w->n_cu;
  const int64_t tiles_per_item = std::max<int64_t>(4, ceil_div(total_units, target_units));
  struct Group { int r, h, split, p0, p1, n_items, rows; int64_t tiles; };
  std::vector<Group> groups[2];
  for (int ri = 0; ri < w->R; ++ri) {
    ReqDesc& r = w->req[ri];
    const bool wide = is_wide(r);
    const int rows = wide ? kShRowsWide : kShRows;
    const int64_t ptiles = ceil_div(r.P, kShKeys);
    int ns = (int)std::min<int64_t>(L.max_splits, std::max<int64_t>(1, ceil_div(ptiles, tiles_per_item)));
    const int64_t chunk_tiles = ceil_div(ptiles, ns);
    ns = (int)ceil_div(ptiles, chunk_tiles);
    r.nsplit = ns;
    const int mt = (int)ceil_div((int64_t)r.W * g, rows);
    for (int s = 0; s < ns; ++s) {
      const int p0 = (int)(s * chunk_tiles * kShKeys);
      const int p1 = (int)std::min<int64_t>(r.P, (s + 1) * chunk_tiles * kShKeys);
      for (int h = 0; h < L.Hkv; ++h)
        groups[wide ? 0 : 1].push_back({ri, h, s, p0, p1, mt, rows, (int64_t)mt * ceil_div(p1 - p0, kShKeys)});
    }
  }
  out.clear();
  n_wide = 0;
  for (int kind = 0; kind < 2; ++kind) {
    std::vector<Group>& gs = groups[kind];
    std::stable_sort(gs.begin(), gs.end(), [](const Group& a, const Group& b) { return a.tiles > b.tiles; });
    constexpr int NX = 8;
    std::vector<std::vector<ShWork>> q(NX);
    std::vector<int64_t> load(NX, 0);
    for (const Group& gr : gs) {
      const int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
      load[x] += gr.tiles;
      for (int m = 0; m < gr.n_items; ++m)
        q[x].push_back({gr.r, gr.h, m * gr.rows, gr.split, gr.p0, gr.p1, 0, 0});
    }
    size_t len = 0;
    for (auto& v : q) len = std::max(len, v.size());
    const size_t before = out.size();
    for (size_t j = 0; j < len; ++j)
      for (int x = 0; x < NX; ++x)
        out.push_back(j < q[x].size() ? q[x][j] : ShWork{-1, 0, 0, 0, 0, 0, 0, 0});
    if (kind == 0) n_wide = (int)(out.size() - before);
  }
}

// Pilot beams of the selection: each pilot contributes one candidate per group of
// 256 / per threads (per a power of two <= top_k, so the contributions of one beam never
// outnumber its pool entries).  Enough pilots for about 8 W candidates, at most kMaxPilots
// beams and kPilotCap candidates per request.  per is at most 256 for the deterministic
// selection, whose slots are ordered by score so that the first beams hold most of the best
// candidates, and at most 64 for the sampled one: there noise decides the slot order, and
// contributions spread over more beams bound the W-th best key far more tightly (kept pool
// 24 K -> 6.8 K entries on the W = K = 512 workload at temperature 1).
int pilot_count(const ReqDesc& d, int max_per, int& per, int max_pilots = kMaxPilots, int cap = kPilotCap) {
  per = 1;
  while (per * 2 <= std::min(d.K, max_per)) per *= 2;
  const int64_t want = ceil_div(8LL * d.W, per);
  const int J = (int)std::min<int64_t>({(int64_t)d.W, (int64_t)max_pilots, (int64_t)(cap / per), want});
  return std::max(1, J);
}

// The general kernels (rows longer than 8192 codes, or W > 1024) take up to kMaxPilotsWide
// pilots and kPilotCapWide candidates, so that requests wider than kPilotCap still get a
// bound (at top_k = 64, W up to about 16000).
void set_pilots(ReqDesc& d, int32_t& pilot_off, int cap) {
  int per;
  d.n_pilot = pilot_count(d, 256, per);
  d.n_pilot_s = pilot_count(d, 64, per);
  const bool wide = cap >= kPilotCapWide;
  d.n_pilot_w = wide ? pilot_count(d, 256, per, kMaxPilotsWide, kPilotCapWide) : d.n_pilot;
  d.n_pilot_ws = wide ? pilot_count(d, 64, per, kMaxPilotsWide, kPilotCapWide) : d.n_pilot_s;
  d.pilot_off = pilot_off;
  pilot_off += cap;
}

// Work list of the generic VALU shared stage: one item per (slot, query head, split).
void build_valu_work(grw_ws* w, std::vector<ShWork>& out) {
  const grw_limits& L = w->lim;
  out.clear();
  for (int ri = 0; ri < w->R; ++ri) {
    ReqDesc& r = w->req[ri];
    const int ns = (int)ceil_div(r.P, kValuMaxKeys);
    r.nsplit = ns;
    for (int b = 0; b < r.W; ++b)
      for (int qh = 0; qh < L.Hq; ++qh)
        for (int s = 0; s < ns; ++s) {
          const int p0 = s * kValuMaxKeys;
          const int p1 = std::min(r.P, (s + 1) * kValuMaxKeys);
          out.push_back({ri, qh, b, s, p0, p1, 0, 0});
        }
  }
}

}  // namespace


// ---------------------------------------------------------------------------------------
// Allocation-free selection of one request (beam_select_noalloc).  Its scratch — the
// request descriptor, slot map, pilot descriptors and buffer, candidate pool and CSR edges,
// survivor counts, bound, step words and flag word — lives in one file-scope device array
// that each GPU holds until the process ends.  Host code never names the array in a device
// context: its device address is looked up once per device with hipGetSymbolAddress and that
// pointer is what the kernels receive.
// ---------------------------------------------------------------------------------------
namespace {

constexpr int kNaMaxW = 1024;                 // the register-resident selection's width limit
constexpr int kNaMaxPool = 512 * 512;         // W * top_k entries of the candidate pool
constexpr int kNaMaxDevices = 64;

// byte offsets inside the scratch array (each 256-byte aligned)
constexpr size_t kNaReq = 0;
constexpr size_t kNaSlotReq = 256;
constexpr size_t kNaPilotDesc = kNaSlotReq + sizeof(int32_t) * kNaMaxW;
constexpr size_t kNaPilotBuf = kNaPilotDesc + sizeof(int32_t) * 4 * kMaxPilots;
constexpr size_t kNaPool = kNaPilotBuf + sizeof(uint64_t) * kPilotCap;
constexpr size_t kNaPoolEdge = kNaPool + sizeof(uint64_t) * kNaMaxPool;
constexpr size_t kNaSurv = kNaPoolEdge + sizeof(int32_t) * kNaMaxPool;
constexpr size_t kNaSync = kNaSurv + sizeof(int32_t) * kNaMaxW;
constexpr size_t kNaWords = kNaSync + sizeof(uint64_t) * kSyncCopies * kSyncStride;   // bound, count, flags
constexpr size_t kNaBytes = kNaWords + 256;
static_assert(kNaSlotReq >= sizeof(ReqDesc) && kNaPilotDesc % 256 == 0 && kNaPilotBuf % 256 == 0 &&
              kNaPool % 256 == 0 && kNaPoolEdge % 256 == 0 && kNaSurv % 256 == 0 && kNaSync % 256 == 0 &&
              kNaWords % 256 == 0, "scratch sections must stay 256-byte aligned");

}  // namespace

// The scratch array itself (about 3.2 MiB per device).
static __device__ __align__(256) uint8_t scratch[kNaBytes];

namespace {

std::mutex g_na_mutex;
void* g_na_ptr[kNaMaxDevices] = {};

// Device address of this device's scratch array (looked up on the first call on the device).
int noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GRW_EDEVICE;
  if (dev < 0 || dev >= kNaMaxDevices) return GRW_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_na_mutex);
  if (g_na_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GRW_EDEVICE;
    g_na_ptr[dev] = p;
  }
  *out = g_na_ptr[dev];
  return GRW_OK;
}

// Per-call set-up inside the scratch: the descriptor, the slot map, the pilot descriptors
// {slot, request, first pilot-buffer entry, threads per group}, and the words that must start
// at zero (bound, pilot count, step words, flags).  One workgroup; a kernel rather than a
// memset so that a captured graph replays it like every other node.
__global__ __launch_bounds__(256) void noalloc_setup_kernel(uint8_t* base, ReqDesc rd, int n_pilot, int per,
                                                            int clear_flags) {
  const int tid = threadIdx.x;
  if (tid == 0) *(ReqDesc*)(base + kNaReq) = rd;
  int32_t* slot_req = (int32_t*)(base + kNaSlotReq);
  for (int i = tid; i < rd.W; i += 256) slot_req[i] = 0;
  int32_t* pd = (int32_t*)(base + kNaPilotDesc);
  for (int j = tid; j < n_pilot; j += 256) {
    pd[4 * j + 0] = j;
    pd[4 * j + 1] = 0;
    pd[4 * j + 2] = j * per;
    pd[4 * j + 3] = 256 / per;
  }
  uint64_t* sync = (uint64_t*)(base + kNaSync);
  for (int i = tid; i < kSyncCopies * kSyncStride; i += 256) sync[i] = 0ull;
  uint32_t* words = (uint32_t*)(base + kNaWords);
  if (tid < 2) words[tid] = 0u;                 // bound, pilot count
  if (tid == 2 && clear_flags) words[2] = 0u;   // flag word (when the caller passes none)
}

}  // namespace

extern "C" {

const char* grw_status_str(int s) {
  switch (s) {
    case GRW_OK: return "ok";
    case GRW_EINVAL: return "invalid argument";
    case GRW_ENOMEM: return "out of memory";
    case GRW_EDEVICE: return "HIP runtime error";
    case GRW_EUNSUPPORTED: return "unsupported shape or dtype";
    case GRW_ESTATE: return "invalid call order (bind a batch first)";
    default: return "unknown status";
  }
}

int grw_ws_create(const grw_limits* limits, grw_ws** out) {
  if (!limits || !out) return GRW_EINVAL;
  *out = nullptr;
  grw_limits L = *limits;
  if (L.max_splits == 0) L.max_splits = 8;
  if (L.max_requests < 1 || L.max_total_beams < 1 || L.max_W < 1 || L.max_K < 1 || L.max_C < 1 ||
      L.max_S < 1 || L.max_P < 1 || L.Hq < 1 || L.Hkv < 1 || L.D < 4 || L.max_splits < 1)
    return GRW_EINVAL;
  if (!dtype_ok(L.q_dtype) || !dtype_ok(L.kv_dtype) || L.q_dtype == GRW_FP8_E4M3) return GRW_EINVAL;
  if (L.max_W > kMaxW || L.max_K > kMaxK || L.max_S > 64 || L.max_splits > 16) return GRW_EUNSUPPORTED;
  if (L.max_W > L.max_total_beams) return GRW_EINVAL;
  if (L.Hq % L.Hkv != 0) return GRW_EINVAL;
  const int g = L.Hq / L.Hkv;
  if (g != 1 && g != 2 && g != 4) return GRW_EUNSUPPORTED;
  const int hd = L.Hkv * L.D;
  if (hd != 128 && hd != 256 && hd != 512 && hd != 1024) return GRW_EUNSUPPORTED;
  if (L.D % 4 != 0 || L.D > 256) return GRW_EUNSUPPORTED;
  if ((uint64_t)L.max_W * (uint64_t)L.max_C >= (1ull << 32)) return GRW_EUNSUPPORTED;

  grw_ws* w = new (std::nothrow) grw_ws();
  if (!w) return GRW_ENOMEM;
  w->lim = L;
  if (hipGetDevice(&w->device) != hipSuccess) { delete w; return GRW_EDEVICE; }
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, w->device) == hipSuccess && cu > 0)
    w->n_cu = cu;
  w->mfma = L.D == 128 && L.q_dtype == GRW_BF16 &&
            (L.kv_dtype == GRW_BF16 || L.kv_dtype == GRW_FP8_E4M3);
  if (!w->mfma && (int64_t)L.max_P > (int64_t)L.max_splits * kValuMaxKeys) {
    delete w;
    return GRW_EUNSUPPORTED;
  }
  const int64_t B = L.max_total_beams;
  const int64_t items = w->mfma ? 2 * mfma_items_bound(L, g) + 8 * 256 + 64
                                : B * L.Hq * L.max_splits;
  w->work_cap = items;
  w->pool_cap = B * (int64_t)L.max_K;
  int st = GRW_OK;
  if (st == GRW_OK) st = dev_alloc(&w->d_req, L.max_requests);
  if (st == GRW_OK) st = dev_alloc(&w->d_slot_req, B);
  if (st == GRW_OK) st = dev_alloc(&w->d_work, items);
  if (st == GRW_OK) st = dev_alloc(&w->d_opart, (int64_t)L.max_splits * B * L.Hq * L.D);
  if (st == GRW_OK) st = dev_alloc(&w->d_lpart, (int64_t)L.max_splits * B * L.Hq);
  if (st == GRW_OK) st = dev_alloc(&w->d_ou, B * L.Hq * L.D);
  if (st == GRW_OK) st = dev_alloc(&w->d_lu, B * L.Hq);
  if (st == GRW_OK) st = dev_alloc(&w->d_pool, w->pool_cap);
  if (st == GRW_OK) st = dev_alloc(&w->d_pool_edge, w->pool_cap);
  if (st == GRW_OK) st = dev_alloc(&w->d_surv_count, B);
  if (st == GRW_OK) st = dev_alloc(&w->d_bound, L.max_requests);
  if (st == GRW_OK) st = dev_alloc(&w->d_pilot_desc, 16 * B);
  if (st == GRW_OK) st = dev_alloc(&w->d_row_lse, B);
  if (st == GRW_OK) st = dev_alloc(&w->d_step_state, (int64_t)L.max_requests);
  if (st == GRW_OK) st = dev_alloc(&w->d_sync, (int64_t)L.max_requests * kSyncCopies * kSyncStride);
  // the general kernels run when rows can be longer than 8192 codes or W larger than 1024
  w->pilot_cap = (L.max_C > kOnePass || L.max_W > 1024) ? kPilotCapWide : kPilotCap;
  if (st == GRW_OK) st = dev_alloc(&w->d_pilot_buf, (int64_t)L.max_requests * w->pilot_cap);
  if (st == GRW_OK) st = dev_alloc(&w->d_flags, 1);
  if (st == GRW_OK) {
    w->stage_bytes = sizeof(ReqDesc) * L.max_requests + sizeof(int32_t) * B + sizeof(ShWork) * items +
                     sizeof(int32_t) * 16 * B;
    if (hipHostMalloc(&w->h_stage, w->stage_bytes, hipHostMallocDefault) != hipSuccess) {
      w->h_stage = nullptr;
      st = GRW_ENOMEM;
    }
  }
  if (st == GRW_OK && (hipEventCreateWithFlags(&w->ev_fork, hipEventDisableTiming) != hipSuccess ||
                       hipEventCreateWithFlags(&w->ev_join, hipEventDisableTiming) != hipSuccess))
    st = GRW_EDEVICE;
  if (st == GRW_OK) {
    if (hipMemset(w->d_bound, 0, sizeof(uint32_t) * L.max_requests) != hipSuccess ||
        hipMemset(w->d_step_state, 0, sizeof(uint32_t) * L.max_requests) != hipSuccess ||
        hipMemset(w->d_sync, 0, sizeof(uint64_t) * L.max_requests * kSyncCopies * kSyncStride) != hipSuccess ||
        hipMemset(w->d_flags, 0, sizeof(int32_t)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
      st = GRW_EDEVICE;
  }
  if (st != GRW_OK) {
    free_all(w);
    delete w;
    return st;
  }
  *out = w;
  return GRW_OK;
}

int grw_ws_destroy(grw_ws* w) {
  if (!w) return GRW_EINVAL;
  (void)hipDeviceSynchronize();
  free_all(w);
  delete w;
  return GRW_OK;
}

namespace {

int bind_batch(grw_ws* w, int32_t n_requests, const int32_t* W_host, const int32_t* K_host, const int32_t* P_host,
               void* stream) {
  const grw_limits& L = w->lim;
  // a failed bind leaves no batch bound: the host mirror below is rewritten before every check
  // has passed, so later step calls must not run against it
  w->bound = false;
  if (n_requests < 1 || n_requests > L.max_requests) return GRW_EINVAL;
  std::vector<ReqDesc> req(n_requests);
  int64_t sumW = 0, kv = 0, pool = 0;
  int maxW = 0, maxK = 0;
  int32_t pilot_off = 0;
  for (int r = 0; r < n_requests; ++r) {
    const int W = W_host[r], K = K_host[r], P = P_host[r];
    if (W < 1 || W > L.max_W || K < 1 || K > L.max_K || P < 1 || P > L.max_P) return GRW_EINVAL;
    ReqDesc& d = req[r];
    d.boff = (int32_t)sumW;
    d.W = W; d.K = K; d.P = P;
    d.Pp = (int32_t)ceil_div(P, kPadP) * kPadP;
    d.nsplit = 1;
    d.kv_off = kv * L.Hkv * L.D;
    d.pool_off = pool;
    set_pilots(d, pilot_off, w->pilot_cap);
    sumW += W;
    kv += d.Pp;
    pool += (int64_t)W * K;
    maxW = std::max(maxW, W);
    maxK = std::max(maxK, K);
  }
  if (sumW > L.max_total_beams || pool > w->pool_cap) return GRW_EINVAL;
  if (!w->mfma) {
    for (const ReqDesc& d : req)
      if (ceil_div(d.P, kValuMaxKeys) > L.max_splits) return GRW_EUNSUPPORTED;
  }
  w->req = req;
  w->R = n_requests;
  w->sumW = (int)sumW;
  std::vector<ShWork> work;
  int n_wide = 0;
  if (w->mfma) build_mfma_work(w, work, n_wide);
  else build_valu_work(w, work);
  if ((int64_t)work.size() > w->work_cap) return GRW_EUNSUPPORTED;
  // one upload: descriptors, slot -> request map, work list
  uint8_t* h = (uint8_t*)w->h_stage;
  ReqDesc* hreq = (ReqDesc*)h;
  int32_t* hslot = (int32_t*)(h + sizeof(ReqDesc) * L.max_requests);
  ShWork* hwork = (ShWork*)(h + sizeof(ReqDesc) * L.max_requests + sizeof(int32_t) * L.max_total_beams);
  int32_t* hpilot = (int32_t*)(hwork + w->work_cap);
  std::memcpy(hreq, w->req.data(), sizeof(ReqDesc) * n_requests);
  // pilot descriptors {slot, request, first pilot-buffer entry, threads per group}, four
  // sets: the register-resident path's deterministic and sampled selections, then the
  // general kernels' deterministic and sampled selections
  int np[4] = {0, 0, 0, 0};
  for (int r = 0; r < n_requests; ++r)
    for (int b = 0; b < req[r].W; ++b) hslot[req[r].boff + b] = r;
  const bool wide = w->pilot_cap >= kPilotCapWide;
  int32_t* hp = hpilot;
  for (int v = 0; v < 4; ++v) {
    int n = 0;
    for (int r = 0; r < n_requests; ++r) {
      int per;
      const int max_per = (v & 1) ? 64 : 256;
      const int J = (v >= 2 && wide) ? pilot_count(req[r], max_per, per, kMaxPilotsWide, kPilotCapWide)
                                     : pilot_count(req[r], max_per, per);
      for (int j = 0; j < J; ++j, ++n) {
        hp[4 * n + 0] = req[r].boff + j;
        hp[4 * n + 1] = r;
        hp[4 * n + 2] = req[r].pilot_off + j * per;
        hp[4 * n + 3] = 256 / per;
      }
    }
    np[v] = n;
    hp += 4 * n;
  }
  const int n_pilots = np[0], n_pilots_s = np[1];
  std::memcpy(hwork, work.data(), sizeof(ShWork) * work.size());
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(w->d_req, hreq, sizeof(ReqDesc) * n_requests, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(w->d_slot_req, hslot, sizeof(int32_t) * sumW, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !work.empty())
    e = hipMemcpyAsync(w->d_work, hwork, sizeof(ShWork) * work.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(w->d_pilot_desc, hpilot, sizeof(int32_t) * 4 * (np[0] + np[1] + np[2] + np[3]),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    w->bound = false;
    return GRW_EDEVICE;
  }
  w->n_work = (int)work.size();
  w->n_wide = n_wide;
  w->n_pilots = n_pilots;
  w->n_pilots_s = n_pilots_s;
  w->n_pilots_w = np[2];
  w->n_pilots_ws = np[3];
  w->maxW = maxW;
  w->maxK = maxK;
  w->bound = true;
  return GRW_OK;
}

}  // namespace

int grw_ws_bind_batch(grw_ws* w, int32_t n_requests, const int32_t* W_host, const int32_t* K_host,
                      const int32_t* P_host, void* stream) {
  if (!w || !W_host || !K_host || !P_host) return GRW_EINVAL;
  try {
    return bind_batch(w, n_requests, W_host, K_host, P_host, stream);
  } catch (const std::bad_alloc&) {   // host work lists of the bind
    w->bound = false;
    return GRW_ENOMEM;
  }
}

int grw_beams_init(grw_ws* w, float* beam_scores, int32_t* beam_node, void* stream) {
  if (!w || !beam_scores || !beam_node) return GRW_EINVAL;
  if (!w->bound) return GRW_ESTATE;
  return hip_status(launch_beams_init(w->d_req, w->d_slot_req, w->sumW, beam_scores, beam_node,
                                      (hipStream_t)stream));
}

int beam_attn_decode(grw_ws* w, const void* q, const void* k_shared, const void* v_shared,
                     const float* k_scale, const float* v_scale, const void* k_unshared,
                     const void* v_unshared, const int32_t* parent_idx, int32_t step,
                     float* out, void* stream) {
  return beam_attn_decode_stages(w, q, k_shared, v_shared, k_scale, v_scale, k_unshared, v_unshared,
                                 parent_idx, step, out, 7, stream);
}

namespace {

// Validates the attention call and fills its kernel arguments.
int attn_args(grw_ws* w, const void* q, const void* k_shared, const void* v_shared, const float* k_scale,
              const float* v_scale, const void* k_unshared, const void* v_unshared,
              const int32_t* parent_idx, int32_t step, float* out, AttnArgs& a) {
  if (!w) return GRW_EINVAL;
  if (!w->bound) return GRW_ESTATE;
  const grw_limits& L = w->lim;
  if (!q || !k_shared || !v_shared || !k_unshared || !v_unshared || !parent_idx || !out)
    return GRW_EINVAL;
  const bool fp8 = L.kv_dtype == GRW_FP8_E4M3;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return GRW_EINVAL;
  if (step < 0 || step >= L.max_S) return GRW_EINVAL;
  a = AttnArgs{};
  a.req = w->d_req;
  a.slot_req = w->d_slot_req;
  a.q = q;
  a.k_shared = k_shared;
  a.v_shared = v_shared;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.k_unshared = k_unshared;
  a.v_unshared = v_unshared;
  a.parent_idx = parent_idx;
  a.step = step;
  a.out = out;
  a.opart = w->d_opart;
  a.lpart = w->d_lpart;
  a.ou = w->d_ou;
  a.lu = w->d_lu;
  a.flags = w->d_flags;
  a.sumW = w->sumW;
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.D = L.D;
  a.g = L.Hq / L.Hkv;
  a.q_dtype = L.q_dtype;
  a.kv_dtype = L.kv_dtype;
  return GRW_OK;
}

hipError_t launch_shared_stage(grw_ws* w, const AttnArgs& a, hipStream_t s) {
  if (!w->mfma) return launch_attn_shared_valu(a, w->d_work, w->n_work, s);
  hipError_t e = launch_attn_shared_split(a, w->d_work, w->n_wide, s);
  if (e == hipSuccess) e = launch_attn_shared_mfma(a, w->d_work + w->n_wide, w->n_work - w->n_wide, s);
  return e;
}

}  // namespace

int beam_attn_decode_stages(grw_ws* w, const void* q, const void* k_shared, const void* v_shared,
                            const float* k_scale, const float* v_scale, const void* k_unshared,
                            const void* v_unshared, const int32_t* parent_idx, int32_t step,
                            float* out, int32_t stages, void* stream) {
  if (stages < 1 || stages > 7) return GRW_EINVAL;
  AttnArgs a;
  const int st = attn_args(w, q, k_shared, v_shared, k_scale, v_scale, k_unshared, v_unshared, parent_idx,
                           step, out, a);
  if (st != GRW_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (stages & GRW_STAGE_SHARED) e = launch_shared_stage(w, a, s);
  const int um = stages & (GRW_STAGE_UNSHARED | GRW_STAGE_MERGE);
  if (e == hipSuccess && um == (GRW_STAGE_UNSHARED | GRW_STAGE_MERGE)) {
    e = launch_attn_unshared_merge(a, s);        // merge fused into the unshared epilogue
  } else {
    if (e == hipSuccess && (stages & GRW_STAGE_UNSHARED)) e = launch_attn_unshared(a, s);
    if (e == hipSuccess && (stages & GRW_STAGE_MERGE)) e = launch_attn_merge(a, s);
  }
  return hip_status(e);
}

int beam_attn_decode_overlap(grw_ws* w, const void* q, const void* k_shared, const void* v_shared,
                             const float* k_scale, const float* v_scale, const void* k_unshared,
                             const void* v_unshared, const int32_t* parent_idx, int32_t step,
                             float* out, void* stream, void* side_stream) {
  if (!side_stream || side_stream == stream) return GRW_EINVAL;
  AttnArgs a;
  const int st = attn_args(w, q, k_shared, v_shared, k_scale, v_scale, k_unshared, v_unshared, parent_idx,
                           step, out, a);
  if (st != GRW_OK) return st;
  hipStream_t s = (hipStream_t)stream, side = (hipStream_t)side_stream;
  // fork: the unshared stage waits for what `stream` already holds (the parent pointers)
  hipError_t e = hipEventRecord(w->ev_fork, s);
  if (e == hipSuccess) e = hipStreamWaitEvent(side, w->ev_fork, 0);
  if (e == hipSuccess) e = launch_attn_unshared(a, side);
  if (e == hipSuccess) e = hipEventRecord(w->ev_join, side);
  if (e == hipSuccess) e = launch_shared_stage(w, a, s);
  // join: the merge needs both partials
  if (e == hipSuccess) e = hipStreamWaitEvent(s, w->ev_join, 0);
  if (e == hipSuccess) e = launch_attn_merge(a, s);
  return hip_status(e);
}

namespace {

// One selection step, deterministic (noise == NULL) or Gumbel-sampled.
int select_step(grw_ws* w, const float* logprobs, bool raw_logits, const float* noise, float temperature,
                const float* beam_scores, const int32_t* beam_node, const int32_t* trie_row_ptr,
                const int32_t* trie_code, int32_t trie_n_internal, int32_t W, int32_t K, int32_t C,
                int32_t* out_token, int32_t* out_parent, float* out_score, int32_t* out_node, void* stream,
                const int32_t* dense_slot = nullptr, const uint32_t* dense_mask = nullptr, bool fanout = false) {
  if (!w) return GRW_EINVAL;
  if (!w->bound) return GRW_ESTATE;
  const grw_limits& L = w->lim;
  if (!logprobs || !beam_scores || !out_token || !out_parent || !out_score || !out_node)
    return GRW_EINVAL;
  const bool trie = trie_row_ptr != nullptr || trie_code != nullptr;
  if (trie && (!trie_row_ptr || !trie_code || !beam_node || trie_n_internal < 1)) return GRW_EINVAL;
  if (W != w->maxW || K != w->maxK) return GRW_EINVAL;
  if (C < 1 || C > L.max_C) return GRW_EINVAL;
  if ((uint64_t)w->maxW * (uint64_t)C >= (1ull << 32)) return GRW_EUNSUPPORTED;
  if ((const void*)out_score == (const void*)beam_scores || (const void*)out_node == (const void*)beam_node)
    return GRW_EINVAL;
  if ((dense_slot != nullptr) != (dense_mask != nullptr) || (dense_slot && !trie)) return GRW_EINVAL;
  // a fan-out wider than kMaxK keeps the prompt beam's whole row in the request's pool region
  if (fanout && w->maxW > kMaxK)
    for (int r = 0; r < w->R; ++r)
      if (w->req[r].W > kMaxK && (int64_t)C > (int64_t)w->req[r].W * w->req[r].K) return GRW_EUNSUPPORTED;
  SelArgs a{};
  a.req = w->d_req;
  a.slot_req = w->d_slot_req;
  a.logprobs = logprobs;
  a.noise = noise;
  a.temp = noise != nullptr ? temperature : 0.0f;
  a.row_lse = raw_logits ? w->d_row_lse : nullptr;
  a.lse_ready = select_fused_ok(C, w->maxW) ? 0 : 1;
  a.scores = beam_scores;
  a.nodes = beam_node;
  a.row_ptr = trie ? trie_row_ptr : nullptr;
  a.code = trie ? trie_code : nullptr;
  a.n_internal = trie_n_internal;
  a.dense_slot = trie ? dense_slot : nullptr;
  a.dense_mask = trie ? dense_mask : nullptr;
  a.mask_words = (C + 31) / 32;
  a.fanout = fanout ? 1 : 0;
  a.C = C;
  a.sumW = w->sumW;
  a.R = w->R;
  a.pool = w->d_pool;
  a.surv_count = w->d_surv_count;
  a.pool_edge = w->d_pool_edge;
  a.bound = w->d_bound;
  if (select_fused_ok(C, w->maxW)) {
    a.pilot_desc = w->d_pilot_desc + (noise != nullptr ? 4 * w->n_pilots : 0);
    a.n_pilots = noise != nullptr ? w->n_pilots_s : w->n_pilots;
  } else {
    a.pilot_desc = w->d_pilot_desc + 4 * (w->n_pilots + w->n_pilots_s) + (noise != nullptr ? 4 * w->n_pilots_w : 0);
    a.n_pilots = noise != nullptr ? w->n_pilots_ws : w->n_pilots_w;
  }
  a.pilot_buf = w->d_pilot_buf;
  a.pilot_count = w->d_step_state;
  a.sync = w->d_sync;
  a.wait_limit = w->wait_limit;
  a.out_token = out_token;
  a.out_parent = out_parent;
  a.out_score = out_score;
  a.out_node = out_node;
  a.flags = w->d_flags;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (select_fused_ok(C, w->maxW)) {
    e = launch_select_fused(a, s);
  } else {
    e = launch_select_topk(a, s);
    if (e == hipSuccess) e = launch_select_global(a, s);
  }
  return hip_status(e);
}

}  // namespace

int beam_select(grw_ws* w, const float* logprobs, const float* beam_scores, const int32_t* beam_node,
                const int32_t* trie_row_ptr, const int32_t* trie_code, int32_t trie_n_internal,
                int32_t W, int32_t K, int32_t C, int32_t* out_token, int32_t* out_parent,
                float* out_score, int32_t* out_node, void* stream) {
  return select_step(w, logprobs, false, nullptr, 0.0f, beam_scores, beam_node, trie_row_ptr, trie_code,
                     trie_n_internal, W, K, C, out_token, out_parent, out_score, out_node, stream);
}

int beam_select_ex(grw_ws* w, const float* input, const float* beam_scores, const int32_t* beam_node,
                   const grw_trie* trie, const grw_select_opts* opts, int32_t W, int32_t K, int32_t C,
                   int32_t* out_token, int32_t* out_parent, float* out_score, int32_t* out_node, void* stream) {
  const float* noise = opts ? opts->noise : nullptr;
  const float temperature = opts ? opts->temperature : 0.0f;
  if (opts && opts->raw_logits != 0 && opts->raw_logits != 1) return GRW_EINVAL;
  if (opts && opts->first_step_fanout != 0 && opts->first_step_fanout != 1) return GRW_EINVAL;
  if (noise && (!(temperature >= 0.0f) || !std::isfinite(temperature))) return GRW_EINVAL;
  return select_step(w, input, opts && opts->raw_logits, noise, temperature, beam_scores, beam_node,
                     trie ? trie->row_ptr : nullptr, trie ? trie->code : nullptr, trie ? trie->n_internal : 0,
                     W, K, C, out_token, out_parent, out_score, out_node, stream,
                     trie ? trie->dense_slot : nullptr, trie ? trie->dense_mask : nullptr,
                     opts && opts->first_step_fanout);
}

int grw_trie_dense_build(const int32_t* row_ptr, const int32_t* code, int32_t n_internal, int32_t C,
                         int32_t min_fanout, int32_t* dense_slot, uint32_t* dense_mask, int32_t* n_dense) {
  if (!row_ptr || !code || !dense_slot || !n_dense || n_internal < 1 || C < 1 || min_fanout < 1)
    return GRW_EINVAL;
  const int64_t words = (C + 31) / 32;
  int32_t n = 0;
  for (int32_t v = 0; v < n_internal; ++v) {
    const int64_t beg = row_ptr[v], end = row_ptr[v + 1];
    if (beg < 0 || end < beg) return GRW_EINVAL;
    dense_slot[v] = end - beg >= min_fanout ? n++ : -1;
  }
  *n_dense = n;
  if (!dense_mask) return GRW_OK;   // count only
  std::memset(dense_mask, 0, sizeof(uint32_t) * words * n);
  for (int32_t v = 0; v < n_internal; ++v) {
    if (dense_slot[v] < 0) continue;
    uint32_t* m = dense_mask + words * dense_slot[v];
    for (int64_t e = row_ptr[v]; e < row_ptr[v + 1]; ++e) {
      const int32_t c = code[e];
      if (c < 0 || c >= C) return GRW_EINVAL;
      m[c >> 5] |= 1u << (c & 31);
    }
  }
  return GRW_OK;
}

int grw_plan_batches(int32_t n, const int32_t* W, int32_t slot_budget, int32_t max_requests,
                     int32_t* batch_of, int32_t* n_batches) {
  if (n < 0 || !n_batches || slot_budget < 1 || max_requests < 1) return GRW_EINVAL;
  if (n > 0 && (!W || !batch_of)) return GRW_EINVAL;
  for (int32_t i = 0; i < n; ++i)
    if (W[i] < 1 || W[i] > slot_budget) return GRW_EINVAL;
  *n_batches = 0;
  if (n == 0) return GRW_OK;
  // Max tree over batches 0..n-1 (at most n open): a leaf holds the batch's free rows, or -1
  // once it holds max_requests requests.  Unopened batches hold the whole budget, so the
  // leftmost leaf with room for a request is an open batch or the next one to open.
  int64_t size = 1;
  while (size < n) size <<= 1;
  std::vector<int32_t> tree, count;
  try {
    tree.assign(2 * (size_t)size, slot_budget);
    count.assign((size_t)n, 0);
  } catch (const std::bad_alloc&) {
    return GRW_ENOMEM;
  }
  int32_t opened = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t w = W[i];
    int64_t v = 1;
    while (v < size) v = tree[2 * v] >= w ? 2 * v : 2 * v + 1;
    const int32_t b = (int32_t)(v - size);   // b <= opened <= i < n: batch `opened` is still empty
    batch_of[i] = b;
    opened = std::max(opened, b + 1);
    const int32_t rows = tree[v] - w;
    tree[v] = ++count[b] >= max_requests ? -1 : rows;
    for (v >>= 1; v >= 1; v >>= 1) tree[v] = std::max(tree[2 * v], tree[2 * v + 1]);
  }
  *n_batches = opened;
  return GRW_OK;
}

int beam_select_logits(grw_ws* w, const float* logits, const float* noise, float temperature,
                       const float* beam_scores, const int32_t* beam_node, const int32_t* trie_row_ptr,
                       const int32_t* trie_code, int32_t trie_n_internal, int32_t W, int32_t K,
                       int32_t C, int32_t* out_token, int32_t* out_parent, float* out_score,
                       int32_t* out_node, void* stream) {
  if (noise && (!(temperature >= 0.0f) || !std::isfinite(temperature))) return GRW_EINVAL;
  return select_step(w, logits, true, noise, temperature, beam_scores, beam_node, trie_row_ptr, trie_code,
                     trie_n_internal, W, K, C, out_token, out_parent, out_score, out_node, stream);
}

int beam_select_gumbel(grw_ws* w, const float* logprobs, const float* noise, float temperature,
                       const float* beam_scores, const int32_t* beam_node, const int32_t* trie_row_ptr,
                       const int32_t* trie_code, int32_t trie_n_internal, int32_t W, int32_t K,
                       int32_t C, int32_t* out_token, int32_t* out_parent, float* out_score,
                       int32_t* out_node, void* stream) {
  if (!noise || !(temperature >= 0.0f) || !std::isfinite(temperature)) return GRW_EINVAL;
  return select_step(w, logprobs, false, noise, temperature, beam_scores, beam_node, trie_row_ptr, trie_code,
                     trie_n_internal, W, K, C, out_token, out_parent, out_score, out_node, stream);
}

int grw_backtrack(grw_ws* w, const int32_t* tokens, const int32_t* parents, int32_t S,
                  int32_t* sid_out, void* stream) {
  if (!w || !tokens || !parents || !sid_out) return GRW_EINVAL;
  if (!w->bound) return GRW_ESTATE;
  if (S < 1 || S > w->lim.max_S) return GRW_EINVAL;
  return hip_status(launch_backtrack(w->d_req, w->d_slot_req, w->sumW, tokens, parents, S, sid_out,
                                     (hipStream_t)stream));
}

int grw_ws_error(grw_ws* w, void* stream, int32_t* flags) {
  if (!w || !flags) return GRW_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  int32_t v = 0;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(&v, w->d_flags, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(w->d_flags, 0, sizeof(int32_t));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  *flags = v;
  return hip_status(e);
}

int grw_ws_pool_size(grw_ws* w, int32_t r, void* stream, int64_t* pool_size) {
  if (!w || !pool_size) return GRW_EINVAL;
  if (!w->bound) return GRW_ESTATE;
  if (r < 0 || r >= w->R) return GRW_EINVAL;
  const ReqDesc& d = w->req[r];
  std::vector<int32_t> cnt(d.W);
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess)
    e = hipMemcpy(cnt.data(), w->d_surv_count + d.boff, sizeof(int32_t) * d.W, hipMemcpyDeviceToHost);
  int64_t n = 0;
  for (int32_t c : cnt) n += c;
  *pool_size = n;
  return hip_status(e);
}

int grw_ws_set_wait_limit(grw_ws* w, int32_t polls) {
  if (!w || polls < 0) return GRW_EINVAL;
  w->wait_limit = polls;
  return GRW_OK;
}

int grw_ws_splits(const grw_ws* w, int32_t r, int32_t* n_splits) {
  if (!w || !n_splits) return GRW_EINVAL;
  if (!w->bound) return GRW_ESTATE;
  if (r < 0 || r >= w->R) return GRW_EINVAL;
  *n_splits = w->req[r].nsplit;
  return GRW_OK;
}


int beam_select_noalloc(const float* logprobs, const float* beam_scores, const int32_t* beam_node,
                        const int32_t* trie_row_ptr, const int32_t* trie_code, int32_t trie_n_internal,
                        int32_t W, int32_t K, int32_t C, int32_t* out_token, int32_t* out_parent,
                        float* out_score, int32_t* out_node, int32_t* device_flags, void* stream) {
  if (!logprobs || !beam_scores || !out_token || !out_parent || !out_score || !out_node) return GRW_EINVAL;
  const bool trie = trie_row_ptr != nullptr || trie_code != nullptr;
  if (trie && (!trie_row_ptr || !trie_code || !beam_node || trie_n_internal < 1)) return GRW_EINVAL;
  if (W < 1 || K < 1 || C < 1) return GRW_EINVAL;
  if ((const void*)out_score == (const void*)beam_scores ||
      (beam_node && (const void*)out_node == (const void*)beam_node))
    return GRW_EINVAL;
  if (W > kNaMaxW || C > kOnePass || K > kMaxK || (int64_t)W * K > kNaMaxPool || !select_fused_ok(C, W))
    return GRW_EUNSUPPORTED;
  void* sp = nullptr;
  const int st = noalloc_scratch(&sp);
  if (st != GRW_OK) return st;
  uint8_t* base = (uint8_t*)sp;
  ReqDesc rd{};
  rd.boff = 0;
  rd.W = W;
  rd.K = K;
  rd.P = 1;
  rd.Pp = kPadP;
  rd.nsplit = 1;
  int per = 1;
  rd.n_pilot = pilot_count(rd, 256, per);
  int per_s = 1;
  rd.n_pilot_s = pilot_count(rd, 64, per_s);
  rd.n_pilot_w = rd.n_pilot;
  rd.n_pilot_ws = rd.n_pilot_s;
  rd.pilot_off = 0;
  hipStream_t s = (hipStream_t)stream;
  noalloc_setup_kernel<<<1, 256, 0, s>>>(base, rd, rd.n_pilot, per, device_flags == nullptr ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return GRW_EDEVICE;
  uint32_t* words = (uint32_t*)(base + kNaWords);
  SelArgs a{};
  a.req = (const ReqDesc*)(base + kNaReq);
  a.slot_req = (const int32_t*)(base + kNaSlotReq);
  a.logprobs = logprobs;
  a.noise = nullptr;
  a.temp = 0.0f;
  a.row_lse = nullptr;
  a.lse_ready = 0;
  a.scores = beam_scores;
  a.nodes = beam_node;
  a.row_ptr = trie ? trie_row_ptr : nullptr;
  a.code = trie ? trie_code : nullptr;
  a.n_internal = trie_n_internal;
  a.mask_words = (C + 31) / 32;
  a.C = C;
  a.sumW = W;
  a.R = 1;
  a.pool = (uint64_t*)(base + kNaPool);
  a.surv_count = (int32_t*)(base + kNaSurv);
  a.pool_edge = (int32_t*)(base + kNaPoolEdge);
  a.bound = words;
  a.pilot_desc = (const int32_t*)(base + kNaPilotDesc);
  a.n_pilots = rd.n_pilot;
  a.pilot_buf = (uint64_t*)(base + kNaPilotBuf);
  a.pilot_count = words + 1;
  a.sync = (uint64_t*)(base + kNaSync);
  a.wait_limit = kBoundSpin;
  a.out_token = out_token;
  a.out_parent = out_parent;
  a.out_score = out_score;
  a.out_node = out_node;
  a.flags = device_flags != nullptr ? device_flags : (int32_t*)(words + 2);
  return hip_status(launch_select_fused(a, s));
}

}  // extern "C"
