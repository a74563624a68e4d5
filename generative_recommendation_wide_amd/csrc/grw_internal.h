// Internal declarations shared by the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/grw.h"

namespace grw {

// Per-request descriptor, uploaded once per bound batch.
struct ReqDesc {
  int32_t boff;      // first global beam slot of the request
  int32_t W, K, P;   // beam width, top_k, prompt length
  int32_t Pp;        // prompt length padded to a multiple of 64 (storage rows)
  int32_t nsplit;    // shared-stage partial results of this request
  int64_t kv_off;    // element offset of the request's prompt block in k_shared / v_shared
  int64_t pool_off;  // first candidate-pool entry of the request (W * min(K, C_max) entries)
  int32_t n_pilot;   // pilot beams of the selection (slots boff .. boff + n_pilot - 1)
  int32_t n_pilot_s; // pilot beams of the sampled (Gumbel) selection
  int32_t pilot_off; // first pilot-buffer entry of the request
  int32_t n_pilot_w;   // pilot beams of the general kernels (rows longer than 8192 codes or
  int32_t n_pilot_ws;  //   W > 1024), deterministic and sampled: up to kPilotCapWide entries
  int32_t pad_;
};

// One shared-stage workgroup: query rows [m0, m0 + rows) of kv head h of request r,
// prompt tokens [p0, p1) written as partial `split`.  r < 0 is a no-op (XCD padding).
struct ShWork {
  int32_t r, h, m0, split;
  int32_t p0, p1, pad0, pad1;
};

// tile sizes of the MFMA shared-stage kernel
constexpr int kShRows = 128;   // query rows per workgroup (4 waves x 32 rows)
constexpr int kShRowsWide = 256;   // query rows per workgroup of the 8-wave bf16 kernel
constexpr int kShKeys = 64;    // prompt keys per LDS tile
constexpr int kPadP = 64;      // prompt storage padding
constexpr int kValuRows = 1;   // the generic VALU shared stage handles one (slot, head) row
constexpr int kValuMaxKeys = 2048;  // keys per split of the VALU shared stage

// selection limits
constexpr int kSelCap = 4096;      // LDS candidate buffer of the per-beam top-k (entries)
constexpr int kSelChunk = 1024;    // candidates appended per round (256 threads x 4)
constexpr int kMaxK = kSelCap - kSelChunk - 1024;   // 2048
constexpr int kMaxW = 8192;        // final sort capacity of the global select
constexpr int kRegC = 32;          // candidates per thread of the one-pass per-beam path
constexpr int kOnePass = 256 * kRegC;   // rows up to this length take the one-pass path
constexpr int kMaxPilots = 64;     // pilot beams per request
constexpr int kPilotCap = 4096;    // pilot candidates per request
constexpr int kMaxPilotsWide = 1024;    // pilot beams per request on the general kernels
constexpr int kPilotCapWide = 16384;    // pilot candidates per request on the general kernels
constexpr int kSyncCopies = 32;    // copies of a request's step-state word (spread polling)
constexpr int kSyncStride = 32;    // words between copies (256 bytes)
constexpr int kBoundSpin = 1 << 18;   // default polls of a beam workgroup waiting for its bound
constexpr int kHistBins = 4096;    // survivor histogram bins of the global select
constexpr int kBinCap = 1024;      // largest histogram bin the global select ranks in place

struct AttnArgs {
  const ReqDesc* req;
  const int32_t* slot_req;
  const void* q;
  const void* k_shared;
  const void* v_shared;
  const float* k_scale;
  const float* v_scale;
  const void* k_unshared;
  const void* v_unshared;
  const int32_t* parent_idx;
  int32_t step;
  float* out;
  float* opart;     // [max_splits][sumW][Hq][D]
  float* lpart;     // [max_splits][sumW][Hq]
  float* ou;        // [sumW][Hq][D]
  float* lu;        // [sumW][Hq]
  int32_t* flags;
  int32_t sumW, Hq, Hkv, D, g;
  int32_t q_dtype, kv_dtype;
};

struct SelArgs {
  const ReqDesc* req;
  const int32_t* slot_req;
  const float* logprobs;
  const float* noise;       // [sumW][C] Gumbel draws of the sampled selection, or NULL
  float temp;               // its temperature (>= 0)
  float* row_lse;           // [sumW] row lse when logprobs holds raw logits, else NULL
  int32_t lse_ready;        // 1: row_lse is filled before the select kernels run
  const float* scores;
  const int32_t* nodes;
  const int32_t* row_ptr;   // NULL: unconstrained
  const int32_t* code;
  int32_t n_internal;
  const int32_t* dense_slot;    // [n_internal] mask index of each node or -1; NULL: CSR only
  const uint32_t* dense_mask;   // [n_dense][mask_words] child bit masks
  int32_t mask_words;           // (C + 31) / 32
  int32_t fanout;               // 1: first-step fan-out (only each request's first slot expands,
                                //    keeping its top W_r candidates instead of top_k)
  int32_t C;
  int32_t sumW, R;
  uint64_t* pool;           // per request: W_r regions of K_r entries (one per beam slot)
  int32_t* surv_count;      // [sumW] entries in each beam's pool region
  int32_t* pool_edge;       // CSR edge of each pool entry (fused step with a trie)
  uint32_t* bound;          // [R] ordered-key lower bound of the W_r-th best key
  const int32_t* pilot_desc;   // [n_pilots][4] beam slot, request, first pilot-buffer entry,
                               // threads per group, of each pilot workgroup
  int32_t n_pilots;
  uint64_t* pilot_buf;      // [R][pilot capacity] pilot candidates
  uint32_t* pilot_count;    // [R] pilots finished this step
  int32_t wait_limit;       // polls before a waiting beam workgroup proceeds without the bound
  uint64_t* sync;           // [R][kSyncCopies] words kSyncStride apart: the request's step
                            //     word for beam workgroups that wait inside the pilot +
                            //     per-beam kernel (top bit: the bound, in the low 32 bits, is
                            //     published); cleared by the W-of-pool stage
  int32_t* out_token;
  int32_t* out_parent;
  float* out_score;
  int32_t* out_node;
  int32_t* flags;
};

// launchers (defined next to their kernels)
hipError_t launch_attn_shared_mfma(const AttnArgs& a, const ShWork* work, int n_work,
                                   hipStream_t s);
hipError_t launch_attn_shared_valu(const AttnArgs& a, const ShWork* work, int n_work,
                                   hipStream_t s);
hipError_t launch_attn_shared_split(const AttnArgs& a, const ShWork* work, int n_work, hipStream_t s);
hipError_t launch_attn_unshared(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_merge(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_unshared_merge(const AttnArgs& a, hipStream_t s);
hipError_t launch_select_topk(const SelArgs& a, hipStream_t s);
hipError_t launch_select_global(const SelArgs& a, hipStream_t s);
bool select_fused_ok(int C, int max_W);
hipError_t launch_select_fused(const SelArgs& a, hipStream_t s);
hipError_t launch_beams_init(const ReqDesc* req, const int32_t* slot_req, int32_t sumW,
                             float* scores, int32_t* nodes, hipStream_t s);
hipError_t launch_backtrack(const ReqDesc* req, const int32_t* slot_req, int32_t sumW,
                            const int32_t* tokens, const int32_t* parents, int32_t S,
                            int32_t* sid, hipStream_t s);
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s);

}  // namespace grw
