// Shared stage of beam attention (xLLM generative-recommendation design doc, section 4.2.2,
// stage 1): every beam's queries attend to the request's prompt KV only, producing a
// normalised partial output and its log-sum-exp.  The prompt KV is stored once per
// request (section 4.2.1) and each tile of it is streamed from HBM into LDS once per
// workgroup, where it is reused by 128 query rows (64 beams x 2 heads for grouped heads
// of 2); workgroups of one (request, kv head) are placed on one XCD so their repeated
// tile reads hit that XCD's L2 rather than HBM.
//
// MFMA path (D = 128, bf16 queries, bf16 or fp8 KV): per wave 32 query rows,
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys x queries), so each lane owns one
//   query column and the row max / sum need only one cross-lane step;
//   O^T += V^T P^T with the same instruction, P kept in registers (the key order inside a
//   16-key step is permuted identically in V^T and P^T, which leaves the sum unchanged).
// fp8 codes are widened to bf16 exactly while being written to LDS; the key scale joins
// the softmax scale and the value scale multiplies the output.
#include "device_common.h"
#include "grw_internal.h"

namespace grw {

namespace {

constexpr int DH = 128;
constexpr int NT = kShKeys;            // 64 keys per tile
constexpr int KS = DH + 8;             // LDS row stride (bf16) of the K tile: 272 B
constexpr int VS = NT + 4;             // LDS row stride (bf16) of the V^T tile: 136 B
constexpr int K_TILE = NT * KS;        // bf16 elements
constexpr float kRescale = 8.0f;       // lazy-rescale margin of the running max (log2 units)
constexpr int V_TILE = DH * VS;

// Register staging of one tile on its way from global memory to LDS.
// bf16: K 4 x 16 B per thread, V^T 4 x 16 B; fp8: 2 + 2 x 16 B (widened to bf16 on store).
template <bool FP8>
struct KRegs {
  u32x4 k[FP8 ? 2 : 4];
};
template <bool FP8>
struct VRegs {
  u32x4 v[FP8 ? 2 : 4];
};

template <bool FP8>
__device__ __forceinline__ void load_k(KRegs<FP8>& t, const uint8_t* kb, int p, int tid) {
  if constexpr (!FP8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int key = c >> 4, dc = c & 15;   // 16 chunks of 8 bf16 per key row
      t.k[i] = *(const u32x4*)(kb + ((size_t)(p + key) * DH + dc * 8) * 2);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int key = c >> 3, dc = c & 7;    // 8 chunks of 16 codes per key row
      t.k[i] = *(const u32x4*)(kb + (size_t)(p + key) * DH + dc * 16);
    }
  }
}

template <bool FP8>
__device__ __forceinline__ void load_v(VRegs<FP8>& t, const uint8_t* vb, int p, int Pp, int tid) {
  if constexpr (!FP8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int d = c >> 3, kc = c & 7;      // 8 chunks of 8 keys per V^T row
      t.v[i] = *(const u32x4*)(vb + ((size_t)d * Pp + p + kc * 8) * 2);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int d = c >> 2, kc = c & 3;      // 4 chunks of 16 codes per V^T row
      t.v[i] = *(const u32x4*)(vb + (size_t)d * Pp + p + kc * 16);
    }
  }
}

template <bool FP8>
__device__ __forceinline__ void store_k(const KRegs<FP8>& t, __bf16* sk, int tid) {
  if constexpr (!FP8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int key = c >> 4, dc = c & 15;
      *(u32x4*)(sk + key * KS + dc * 8) = t.k[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int key = c >> 3, dc = c & 7;
      u32x2 a = fp8x4_to_bf16x4(t.k[i].x), b = fp8x4_to_bf16x4(t.k[i].y);
      u32x2 e = fp8x4_to_bf16x4(t.k[i].z), f = fp8x4_to_bf16x4(t.k[i].w);
      u32x4* kd = (u32x4*)(sk + key * KS + dc * 16);
      kd[0] = u32x4{a.x, a.y, b.x, b.y};
      kd[1] = u32x4{e.x, e.y, f.x, f.y};
    }
  }
}

template <bool FP8>
__device__ __forceinline__ void store_v(const VRegs<FP8>& t, __bf16* sv, int tid) {
  if constexpr (!FP8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int d = c >> 3, kc = c & 7;
      u32x2* dst = (u32x2*)(sv + d * VS + kc * 8);   // rows are 8-byte aligned
      dst[0] = u32x2{t.v[i].x, t.v[i].y};
      dst[1] = u32x2{t.v[i].z, t.v[i].w};
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int d = c >> 2, kc = c & 3;
      u32x2* vd = (u32x2*)(sv + d * VS + kc * 16);
      vd[0] = fp8x4_to_bf16x4(t.v[i].x);
      vd[1] = fp8x4_to_bf16x4(t.v[i].y);
      vd[2] = fp8x4_to_bf16x4(t.v[i].z);
      vd[3] = fp8x4_to_bf16x4(t.v[i].w);
    }
  }
}

// S^T = K Q^T for one 64-key tile: two 32-key blocks of 32 queries.
__device__ __forceinline__ void tile_scores(const __bf16* kt, const bf16x8 (&qf)[DH / 16], int l32, int hi,
                                            floatx16& s0, floatx16& s1) {
  s0 = floatx16{};
  s1 = floatx16{};
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks) {
    const bf16x8 a0 = *(const bf16x8*)(kt + l32 * KS + ks * 16 + hi * 8);
    const bf16x8 a1 = *(const bf16x8*)(kt + (32 + l32) * KS + ks * 16 + hi * 8);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], s1, 0, 0, 0);
  }
}

__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                              float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// Maximum of the 32 scores a lane holds for one row (16 of each of two key blocks) as a tree
// of three-input maxima: 18 instructions, 4 dependent steps (a running chain takes 16 steps).
__device__ __forceinline__ float max32(const floatx16& x, const floatx16& y) {
  float t[11];
#pragma unroll
  for (int j = 0; j < 5; ++j) t[j] = vmax(vmax(x[3 * j], x[3 * j + 1]), x[3 * j + 2]);
#pragma unroll
  for (int j = 0; j < 5; ++j) t[5 + j] = vmax(vmax(y[3 * j], y[3 * j + 1]), y[3 * j + 2]);
  t[10] = vmax(x[15], y[15]);
  const float u0 = vmax(vmax(t[0], t[1]), t[2]), u1 = vmax(vmax(t[3], t[4]), t[5]);
  const float u2 = vmax(vmax(t[6], t[7]), t[8]), u3 = vmax(t[9], t[10]);
  return vmax(vmax(vmax(u0, u1), u2), u3);
}

// Store a wave's 32 rows of normalised partial output and their LSE.  The partial output
// goes out through LDS so that every store instruction writes whole rows (512 B per query
// row): written straight from the MFMA layout, each instruction would put 32-byte pieces of
// 32 rows.  Called once every wave is past its last tile (8 KB of smem per wave are free);
// each wave stages its 32 rows x 64 dims (8 KB, 16-byte chunk c of row r at c ^ (r % 16))
// twice.  out_scale multiplies the output (the fp8 V scale, else 1).
__device__ __forceinline__ void store_partial(const AttnArgs& a, const ShWork& wk, const ReqDesc& rd, uint8_t* smem,
                                              const floatx16 (&o)[DH / 32], float m_run, float l_run, bool row_ok,
                                              int slot, int qh, float out_scale) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int g = a.g, Hq = a.Hq, h = wk.h;
  const int nrows = rd.W * g;
  const float l = l_run + lane_xor<32>(l_run);
  const float inv = row_ok ? out_scale / l : 0.0f;
  if (row_ok && hi == 0) a.lpart[((size_t)wk.split * a.sumW + slot) * Hq + qh] = (m_run + fast_log2(l)) * kLn2;
  uint8_t* tb = smem + wave * 8192;
  const int rrow = lane >> 4, rch = lane & 15;   // read side: 4 rows of 16 chunks per instruction
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int db2 = 0; db2 < 2; ++db2) {
      const int db = half * 2 + db2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = db2 * 8 + i * 2 + hi;
        const floatx4 v = {o[db][i * 4 + 0] * inv, o[db][i * 4 + 1] * inv, o[db][i * 4 + 2] * inv,
                           o[db][i * 4 + 3] * inv};
        *(floatx4*)(tb + l32 * 256 + ((ch ^ (l32 & 15)) << 4)) = v;
      }
    }
    __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15);   // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 4 + rrow;
      const floatx4 v = *(const floatx4*)(tb + r * 256 + ((rch ^ (r & 15)) << 4));
      const int mr = wk.m0 + wave * 32 + r;
      if (mr < nrows) {
        const int bb = mr / g;
        const int qq = h * g + (mr - bb * g);
        float* dst = a.opart + (((size_t)wk.split * a.sumW + rd.boff + bb) * Hq + qq) * DH;
        __builtin_nontemporal_store(v, (floatx4*)(dst + half * 64 + rch * 4));   // read back by the next launch only
      }
    }
    __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15);   // reads done before the next half overwrites
    __builtin_amdgcn_wave_barrier();
  }
}

template <bool FP8>
__global__ __launch_bounds__(256, 2) void attn_shared_mfma_kernel(AttnArgs a, const ShWork* __restrict__ work) {
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (K_TILE + V_TILE)];
  const ShWork wk = work[blockIdx.x];
  if (wk.r < 0) return;
  const ReqDesc rd = a.req[wk.r];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int g = a.g, Hq = a.Hq, h = wk.h;
  const int nrows = rd.W * g;

  // this lane's query row (the B-operand column of S^T and of O^T)
  const int mrow = wk.m0 + wave * 32 + l32;
  const bool row_ok = mrow < nrows;
  const int b = row_ok ? mrow / g : 0;
  const int qh = h * g + (row_ok ? mrow - b * g : 0);
  const int slot = rd.boff + b;

  bf16x8 qf[DH / 16];
  {
    const __bf16* qrow = (const __bf16*)a.q + ((size_t)slot * Hq + qh) * DH;
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks) {
      if (row_ok) {
        qf[ks] = *(const bf16x8*)(qrow + ks * 16 + hi * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)0.0f;
      }
    }
  }

  const size_t esz = FP8 ? 1 : 2;
  const uint8_t* kb = (const uint8_t*)a.k_shared + (rd.kv_off + (size_t)h * rd.Pp * DH) * esz;
  const uint8_t* vb = (const uint8_t*)a.v_shared + (rd.kv_off + (size_t)h * DH * rd.Pp) * esz;

  float c = rsqrtf((float)DH) * kLog2e;     // softmax scale in log2 units
  float vscale = 1.0f;
  if constexpr (FP8) {
    c *= a.k_scale[h];
    vscale = a.v_scale[h];
  }

  const int p0 = wk.p0, p1 = wk.p1;
  const int ntiles = (p1 - p0 + NT - 1) / NT;

  // LDS: K tiles [2][NT][KS], then V^T tiles [2][DH][VS], double buffered: tile t+1 is
  // fetched into registers while tile t is consumed, then stored to the other buffer.
  __bf16* const sk0 = smem;
  __bf16* const sv0 = smem + 2 * K_TILE;

  KRegs<FP8> kr;
  VRegs<FP8> vr;
  load_k<FP8>(kr, kb, p0, tid);
  load_v<FP8>(vr, vb, p0, rd.Pp, tid);
  store_k<FP8>(kr, sk0, tid);
  store_v<FP8>(vr, sv0, tid);
  __syncthreads();

  float m_run = -INFINITY;   // running max of scaled scores (identical on both lane halves)
  float l_run = 0.0f;        // this lane's share of the running sum
  floatx16 o[DH / 32];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db) o[db] = floatx16{};

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int p = p0 + t * NT;
    const bool more = t + 1 < ntiles;
    if (more) {
      load_k<FP8>(kr, kb, p + NT, tid);
      load_v<FP8>(vr, vb, p + NT, rd.Pp, tid);
    }
    floatx16 s0, s1;
    __builtin_amdgcn_s_setprio(1);
    tile_scores(sk0 + buf * K_TILE, qf, l32, hi, s0, s1);
    __builtin_amdgcn_s_setprio(0);
    // value k of block kb belongs to key p + kb*32 + (k/4)*8 + hi*4 + k%4
    if (p + NT > p1) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int key = p + (k >> 2) * 8 + hi * 4 + (k & 3);
        if (key >= p1) s0[k] = -INFINITY;
        if (key + 32 >= p1) s1[k] = -INFINITY;
      }
    }
    float mx = max32(s0, s1);
    mx = half_swap_max(mx) * c;
    // Lazy rescale: the running max m_run only moves when some row's tile max exceeds it
    // by more than kRescale (log2 units), so p = 2^(s*c - m_run) <= 2^kRescale and the
    // O / l rescale runs on a few tiles only (wave-uniform branch).
    if (__any(mx > m_run + kRescale)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);   // m_run = -inf -> 0
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DH / 32; ++db) o[db] *= alpha;
      m_run = m_new;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      s0[k] = fast_exp2(fmaf(s0[k], c, -m_run));
      s1[k] = fast_exp2(fmaf(s1[k], c, -m_run));
    }
    // P^T fragments: k-step ks covers 16 keys; lane half `hi` supplies its 8 values
    bf16x8 pb[4];
    pb[0] = pack_bf16x8(s0[0], s0[1], s0[2], s0[3], s0[4], s0[5], s0[6], s0[7]);
    pb[1] = pack_bf16x8(s0[8], s0[9], s0[10], s0[11], s0[12], s0[13], s0[14], s0[15]);
    pb[2] = pack_bf16x8(s1[0], s1[1], s1[2], s1[3], s1[4], s1[5], s1[6], s1[7]);
    pb[3] = pack_bf16x8(s1[8], s1[9], s1[10], s1[11], s1[12], s1[13], s1[14], s1[15]);
    // row sum of the bf16-rounded P (the values the PV product uses), two per instruction
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i], pb[i], 0, 1), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i], pb[i], 2, 3), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i], pb[i], 4, 5), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i], pb[i], 6, 7), ones, l_run, false);
    }

    // O^T += V^T P^T
    const __bf16* vt = sv0 + buf * V_TILE;
    const bool tail = p + NT > p1;   // keys >= p1 in this tile: storage padding or the next split
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb0 = (ks >> 1) * 32 + (ks & 1) * 16 + hi * 4;   // first key of the lane's run
#pragma unroll
      for (int db = 0; db < DH / 32; ++db) {
        const __bf16* row = vt + (db * 32 + l32) * VS;
        const bf16x4 v0 = *(const bf16x4*)(row + kb0);
        const bf16x4 v1 = *(const bf16x4*)(row + kb0 + 8);
        bf16x8 av = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        if (tail) {
          // p = 0 there, but padding may hold any bits (0 * NaN = NaN): those values become 0
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (p + kb0 + (e >> 2) * 8 + (e & 3) >= p1) av[e] = (__bf16)0.0f;
        }
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks], o[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);

    if (more) {
      store_k<FP8>(kr, sk0 + (buf ^ 1) * K_TILE, tid);
      store_v<FP8>(vr, sv0 + (buf ^ 1) * V_TILE, tid);
    }
    __syncthreads();
  }

  __syncthreads();   // every wave is past its last tile: the tile buffers are free
  store_partial(a, wk, rd, (uint8_t*)smem, o, m_run, l_run, row_ok, slot, qh, vscale);
}

// ---------------------------------------------------------------------------------------
// Prompt tiles of the wide-request bf16 path.  Tiles move global -> LDS with
// global_load_lds_dwordx4 (no register staging, no LDS store instructions).  They are
// unpadded and XOR-swizzled so the MFMA operand reads are conflict-free 16-byte reads:
//   K tile   [64 keys][128 d]: 16-byte chunk lc of row r sits at chunk lc ^ (r % 16);
//            row r holds key k_row_key(r), a permutation inside each 32-key block chosen so
//            that the eight P values a lane feeds one PV k-step are eight consecutive keys;
//   V^T tile [128 d][64 keys]: chunk lc of row d sits at chunk lc ^ ((d / 2) % 8).
// ---------------------------------------------------------------------------------------
namespace lds {

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int k_row_key(int r) {
  const int x = r & 31;
  const int i = x >> 3, hh = (x >> 2) & 1, j = x & 3;
  return (r & 32) + (i >> 1) * 16 + hh * 8 + (i & 1) * 4 + j;
}

__device__ __forceinline__ void wait_all_vm() {
  __builtin_amdgcn_s_waitcnt((15 << 8) | (7 << 4) | 0);   // vmcnt(0)
}

}  // namespace lds

// ---------------------------------------------------------------------------------------
// Wide-request bf16 path (W * g > 128 rows): 8 waves and 256 query rows (128 beams x 2
// grouped heads) per workgroup, so each prompt tile read from L2 feeds twice the rows of
// the 4-wave kernel above.  The roles are split: waves 0-3 (score waves) each compute
// S^T = K Q^T and the softmax for 64 rows, and waves 4-7 (product waves) each accumulate
// O^T += V^T P^T for the same 64 rows.  P goes from a score wave to its product wave through LDS (one 8 KB buffer per
// wave pair and tile, in the MFMA B-operand layout, double buffered), with the per-row
// rescale factor when the running max moves.  A score wave and its product wave share a
// SIMD (wave w runs on SIMD w mod 4), so the product wave's MFMAs can run while the score
// wave does its exponentials, and each K or V fragment read from LDS feeds two MFMAs (two
// 32-row blocks) instead of one.  Iteration i: score waves handle tile i, product waves
// tile i - 1; one barrier per iteration.
// ---------------------------------------------------------------------------------------
namespace split {

constexpr int NWAVES = 8;
constexpr int TILE_BYTES = NT * DH * 2;               // 16 KB: one K or V^T tile
constexpr int KRING = 0;                              // K tiles [2]
constexpr int VRING = 2 * TILE_BYTES;                 // V^T tiles [2]
constexpr int P_WAVE = 2 * 4 * 64 * 16;               // P of one score wave: [2 qb][4 ks][64 lanes][16 B]
constexpr int PBUF = 4 * TILE_BYTES;                  // P [2 buffers][4 score waves]
constexpr int ALPHA = PBUF + 2 * 4 * P_WAVE;          // rescale factors [2][4][64] float
constexpr int FLAG = ALPHA + 2 * 4 * 64 * 4;          // rescale flags [2][4] int
constexpr int SMEM_BYTES = FLAG + 2 * 4 * 4;

// Direct-to-LDS loads of one K tile (rows in k_row_key order, swizzled) and one V^T tile:
// each wave moves 2 KB of each, chunks 2 wave and 2 wave + 1.  A lane's byte offsets within
// a tile do not depend on the tile, so they are formed once (TileOffsets); per tile only the
// tile's base address (wave-uniform) moves, and the LDS destinations are scalar.
struct TileOffsets {
  uint32_t k[2], v[2];
};
__device__ __forceinline__ TileOffsets tile_offsets(int wave, int lane, int Pp) {
  TileOffsets t;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = (wave * 2 + i) * 64 + lane;
    const int r = j >> 4, lk = (j & 15) ^ (r & 15);
    t.k[i] = (uint32_t)((lds::k_row_key(r) * DH + lk * 8) * 2);          // < 16 KB
    const int d = j >> 3, lv = (j & 7) ^ ((d >> 1) & 7);
    t.v[i] = (uint32_t)(d * Pp + lv * 8) * 2u;                           // within the prompt block
  }
  return t;
}
__device__ __forceinline__ void issue_k(uint8_t* dst, const uint8_t* kb, int p, int wave, const TileOffsets& t) {
  const uint8_t* base = kb + (size_t)p * (DH * 2);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(base + t.k[i]), (lds::lds_void*)(dst + (wave * 2 + i) * 1024), 16, 0, 0);
}
__device__ __forceinline__ void issue_v(uint8_t* dst, const uint8_t* vb, int p, int wave, const TileOffsets& t) {
  const uint8_t* base = vb + (size_t)p * 2;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(base + t.v[i]), (lds::lds_void*)(dst + (wave * 2 + i) * 1024), 16, 0, 0);
}

// Normalised partial output and LSE of one 32-row block (rows row0 .. row0 + 31 of the
// request's W*g rows, lane l32 holding row row0 + l32 in o), written as whole 512-byte
// rows through the 8 KB LDS buffer tb (16-byte chunk c of row r at c ^ (r % 16)).
__device__ __forceinline__ void store_rows(const AttnArgs& a, const ShWork& wk, const ReqDesc& rd, uint8_t* tb,
                                           const floatx16 (&o)[DH / 32], float m, float l, int row0) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  const int g = a.g, Hq = a.Hq, h = wk.h;
  const int nrows = rd.W * g;
  const int mrow = row0 + l32;
  const bool row_ok = mrow < nrows;
  const float inv = row_ok ? 1.0f / l : 0.0f;
  if (row_ok && hi == 0) {
    const int b = mrow / g;
    a.lpart[((size_t)wk.split * a.sumW + rd.boff + b) * Hq + h * g + (mrow - b * g)] = (m + fast_log2(l)) * kLn2;
  }
  const int rrow = lane >> 4, rch = lane & 15;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int db2 = 0; db2 < 2; ++db2) {
      const int db = half * 2 + db2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = db2 * 8 + i * 2 + hi;
        const floatx4 v = {o[db][i * 4 + 0] * inv, o[db][i * 4 + 1] * inv, o[db][i * 4 + 2] * inv,
                           o[db][i * 4 + 3] * inv};
        *(floatx4*)(tb + l32 * 256 + ((ch ^ (l32 & 15)) << 4)) = v;
      }
    }
    __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = it * 4 + rrow;
      const floatx4 v = *(const floatx4*)(tb + r * 256 + ((rch ^ (r & 15)) << 4));
      const int mr = row0 + r;
      if (mr < nrows) {
        const int bb = mr / g;
        const int qq = h * g + (mr - bb * g);
        float* dst = a.opart + (((size_t)wk.split * a.sumW + rd.boff + bb) * Hq + qq) * DH;
        __builtin_nontemporal_store(v, (floatx4*)(dst + half * 64 + rch * 4));   // read back by the next launch only
      }
    }
    __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15);
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(NWAVES * 64, 1) void attn_shared_split_kernel(AttnArgs a, const ShWork* __restrict__ work) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const ShWork wk = work[blockIdx.x];
  if (wk.r < 0) return;
  const ReqDesc rd = a.req[wk.r];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
  const int l32 = lane & 31, hi = lane >> 5;
  const int g = a.g, Hq = a.Hq, h = wk.h;
  const int nrows = rd.W * g;
  const bool scorer = wave < 4;
  const int sw = wave & 3;                  // the pair: rows wk.m0 + sw * 64 .. + 63
  const uint8_t* kb = (const uint8_t*)a.k_shared + (rd.kv_off + (size_t)h * rd.Pp * DH) * 2;
  const uint8_t* vb = (const uint8_t*)a.v_shared + (rd.kv_off + (size_t)h * DH * rd.Pp) * 2;
  const int p0 = wk.p0, p1 = wk.p1;
  const int ntiles = (p1 - p0 + NT - 1) / NT;
  float* const alpha_s = (float*)(smem + ALPHA);
  int* const flag_s = (int*)(smem + FLAG);

  const TileOffsets toff = tile_offsets(wave, lane, rd.Pp);
  issue_k(smem + KRING, kb, p0, wave, toff);

  if (scorer) {
    // ---------------- score wave: S^T, running max, P ----------------
    // The score products deliver the exponent arguments x = c s - m (log2 units) directly:
    // Q is held pre-scaled by c = log2(e) / sqrt(D) (one bf16 rounding of c q), and a ninth
    // k-step adds -m to every row, its K fragment holding ones in dimensions 0 and 1 and its Q
    // fragment the row's -m_hi, -m_lo.  The running max m is kept as m_hi + m_lo (two bf16
    // values, the sum exact in float), so the m the products subtract is the m of the LSE.
    const float c = rsqrtf((float)DH) * kLog2e;
    bf16x8 qf[2][DH / 16];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int mrow = wk.m0 + sw * 64 + qb * 32 + l32;
      const bool ok = mrow < nrows;
      const int b = ok ? mrow / g : 0;
      const int qh = h * g + (ok ? mrow - b * g : 0);
      const __bf16* qrow = (const __bf16*)a.q + ((size_t)(rd.boff + b) * Hq + qh) * DH;
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) {
        if (ok) {
          const bf16x8 q8 = *(const bf16x8*)(qrow + ks * 16 + hi * 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[qb][ks][e] = (__bf16)((float)q8[e] * c);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[qb][ks][e] = (__bf16)0.0f;
        }
      }
    }
    bf16x8 kone, qm[2];   // the extra k-step's K fragment, and its Q fragment per row block
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kone[e] = (__bf16)((hi == 0 && e < 2) ? 1.0f : 0.0f);
      qm[0][e] = qm[1][e] = (__bf16)0.0f;
    }
    // sets row block qb's subtracted max to (about) m; returns the value subtracted
    auto set_m = [&](int qb, float m) -> float {
      const __bf16 mh = (__bf16)m;
      const __bf16 ml = (__bf16)(m - (float)mh);
      if (hi == 0) {
        qm[qb][0] = (__bf16)(-(float)mh);
        qm[qb][1] = (__bf16)(-(float)ml);
      }
      return (float)mh + (float)ml;
    };
    float m_run[2] = {0.0f, 0.0f};
    for (int i = 0; i <= ntiles; ++i) {
      lds::wait_all_vm();
      __syncthreads();
      const uint8_t* st = smem + KRING + (i & 1) * TILE_BYTES;
      bf16x8 kf[2][2][4];   // [half of D][key block][k-step of the half]
      auto read_kf = [&](int h2) {
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const int lc = 2 * (h2 * 4 + k4) + hi;
          kf[h2][0][k4] = *(const bf16x8*)(st + l32 * 256 + ((lc ^ (l32 & 15)) << 4));
          kf[h2][1][k4] = *(const bf16x8*)(st + (32 + l32) * 256 + ((lc ^ (l32 & 15)) << 4));
        }
      };
      // the first fragments' LDS latency passes while the tile loads are issued
      if (i < ntiles) read_kf(0);
      if (i + 1 < ntiles) issue_k(smem + KRING + ((i + 1) & 1) * TILE_BYTES, kb, p0 + (i + 1) * NT, wave, toff);
      if (i < ntiles) issue_v(smem + VRING + (i & 1) * TILE_BYTES, vb, p0 + i * NT, wave, toff);
      if (i == ntiles) break;
      const int p = p0 + i * NT;
      floatx16 s[2][2];   // [key block][row block]
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[kb2][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kone, qm[qb], floatx16{}, 0, 0, 0);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        if (h2 == 1) read_kf(1);
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              s[kb2][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[h2][kb2][k4], qf[qb][h2 * 4 + k4], s[kb2][qb], 0, 0, 0);
      }
      __builtin_amdgcn_s_setprio(0);
      // value k of key block kb2 is key p + kb2*32 + (k/8)*16 + hi*8 + ((k/4)%2)*4 + k%4
      if (p + NT > p1) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int key = p + ((k >> 3) << 4) + hi * 8 + (((k >> 2) & 1) << 2) + (k & 3);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            if (key >= p1) s[0][qb][k] = -INFINITY;
            if (key + 32 >= p1) s[1][qb][k] = -INFINITY;
          }
        }
      }
      float mx[2];   // the row's largest x in this tile
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float m = max32(s[0][qb], s[1][qb]);
        mx[qb] = half_swap_max(m);
      }
      // Lazy rescale as in the kernels above: m moves when some row's x exceeds kRescale (on
      // the first tile, to the tile max); then x drops by the shift and the product wave
      // scales O and l by 2^-shift.
      const int bi = (i & 1) * 4 + sw;
      const bool resc = i == 0 || __any(mx[0] > kRescale || mx[1] > kRescale);
      if (resc) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float m_new = set_m(qb, m_run[qb] + (i == 0 ? mx[qb] : fmaxf(mx[qb], 0.0f)));
          const float shift = m_new - m_run[qb];
          const float al = i == 0 ? 0.0f : fast_exp2(-shift);
          m_run[qb] = m_new;
          if (hi == 0) alpha_s[bi * 64 + qb * 32 + l32] = al;
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int k = 0; k < 16; ++k) s[kb2][qb][k] -= shift;
        }
      }
      if (lane == 0) flag_s[bi] = resc ? 1 : 0;
      uint8_t* pw = smem + PBUF + bi * P_WAVE;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            float e[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) e[x] = fast_exp2(s[kb2][qb][half * 8 + x]);
            const int ks = kb2 * 2 + half;
            *(bf16x8*)(pw + ((qb * 4 + ks) * 64 + lane) * 16) = pack_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
          }
        }
      }
    }
    __syncthreads();   // every product wave is past its last tile
    if (hi == 0) {
      alpha_s[sw * 64 + l32] = m_run[0];
      alpha_s[sw * 64 + 32 + l32] = m_run[1];
    }
    __syncthreads();
  } else {
    // ---------------- product wave: O^T += V^T P^T, row sums ----------------
    floatx16 o[2][DH / 32];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int db = 0; db < DH / 32; ++db) o[qb][db] = floatx16{};
    float l_run[2] = {0.0f, 0.0f};
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    for (int i = 0; i <= ntiles; ++i) {
      lds::wait_all_vm();
      __syncthreads();
      if (i + 1 < ntiles) issue_k(smem + KRING + ((i + 1) & 1) * TILE_BYTES, kb, p0 + (i + 1) * NT, wave, toff);
      if (i < ntiles) issue_v(smem + VRING + (i & 1) * TILE_BYTES, vb, p0 + i * NT, wave, toff);
      if (i == 0) continue;
      const int bt = ((i - 1) & 1) * 4 + sw;
      if (flag_s[bt]) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float al = alpha_s[bt * 64 + qb * 32 + l32];
          l_run[qb] *= al;
#pragma unroll
          for (int db = 0; db < DH / 32; ++db) o[qb][db] *= al;
        }
      }
      const uint8_t* pp = smem + PBUF + bt * P_WAVE;
      const uint8_t* vt = smem + VRING + ((i - 1) & 1) * TILE_BYTES;
      const int pt = p0 + (i - 1) * NT;          // first key of the tile
      const bool tail = pt + NT > p1;            // wave-uniform: the split's last, partial tile
      bf16x8 pf[2][4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) pf[qb][ks] = *(const bf16x8*)(pp + ((qb * 4 + ks) * 64 + lane) * 16);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        bf16x8 vf[2][DH / 32];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int lc = 2 * (h2 * 2 + k2) + hi;
#pragma unroll
          for (int db = 0; db < DH / 32; ++db) {
            const int d = db * 32 + l32;
            vf[k2][db] = *(const bf16x8*)(vt + d * 128 + ((lc ^ ((d >> 1) & 7)) << 4));
          }
          if (tail) {
            // keys >= p1 (storage padding or the next split) have p = 0, but padding may hold
            // any bits (0 * NaN = NaN): their values become 0.  Chunk lc holds keys 8 lc .. 8 lc + 7.
#pragma unroll
            for (int db = 0; db < DH / 32; ++db)
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (pt + lc * 8 + e >= p1) vf[k2][db][e] = (__bf16)0.0f;
          }
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int db = 0; db < DH / 32; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[k2][db], pf[qb][h2 * 2 + k2], o[qb][db], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
      }
      // row sums of the bf16 P the products used
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[qb][ks], pf[qb][ks], 0, 1), ones, l_run[qb], false);
          l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[qb][ks], pf[qb][ks], 2, 3), ones, l_run[qb], false);
          l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[qb][ks], pf[qb][ks], 4, 5), ones, l_run[qb], false);
          l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[qb][ks], pf[qb][ks], 6, 7), ones, l_run[qb], false);
        }
    }
    __syncthreads();   // every wave is past its last tile: the rings are free
    __syncthreads();   // the score waves' final running maxima are in alpha_s
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m = alpha_s[sw * 64 + qb * 32 + l32];
      const float l = l_run[qb] + lane_xor<32>(l_run[qb]);
      store_rows(a, wk, rd, smem + KRING + sw * TILE_BYTES, o[qb], m, l, wk.m0 + sw * 64 + qb * 32);
    }
  }
}

}  // namespace split


// ---------------------------------------------------------------------------------------
// Generic VALU shared stage: one workgroup per (slot, query head, split), any dtype and
// head dim <= 256.  Used for float32 inputs and shapes the MFMA kernel does not cover.
// Work item fields: r, h = query head, m0 = request-local slot, split, p0, p1.
// ---------------------------------------------------------------------------------------
template <int KVT>
__device__ __forceinline__ float kv_load(const void* base, size_t i) {
  if constexpr (KVT == GRW_F32) return ((const float*)base)[i];
  else if constexpr (KVT == GRW_BF16) return bf16_bits_to_f32(((const uint16_t*)base)[i]);
  else {
    const uint32_t byte = ((const uint8_t*)base)[i];
    return fp8x2_to_f32<false>(byte).x;
  }
}

template <int KVT>
__global__ __launch_bounds__(256) void attn_shared_valu_kernel(AttnArgs a, const ShWork* __restrict__ work) {
  __shared__ float qs[256];
  __shared__ float ss[kValuMaxKeys];
  __shared__ float red[8];
  const ShWork wk = work[blockIdx.x];
  if (wk.r < 0) return;
  const ReqDesc rd = a.req[wk.r];
  const int tid = threadIdx.x, D = a.D, qh = wk.h, hk = qh / a.g;
  const int slot = rd.boff + wk.m0;
  const size_t qi = ((size_t)slot * a.Hq + qh) * D;
  for (int d = tid; d < D; d += 256)
    qs[d] = a.q_dtype == GRW_F32 ? ((const float*)a.q)[qi + d]
                                 : bf16_bits_to_f32(((const uint16_t*)a.q)[qi + d]);
  __syncthreads();
  float c = rsqrtf((float)D) * kLog2e;
  float vscale = 1.0f;
  if (KVT == GRW_FP8_E4M3) {
    c *= a.k_scale[hk];
    vscale = a.v_scale[hk];
  }
  const size_t kbase = rd.kv_off + (size_t)hk * rd.Pp * D;   // [Pp][D]
  const size_t vbase = rd.kv_off + (size_t)hk * D * rd.Pp;   // [D][Pp]
  const int n = wk.p1 - wk.p0;
  float mx = -INFINITY;
  for (int t = tid; t < n; t += 256) {
    const size_t row = kbase + (size_t)(wk.p0 + t) * D;
    float s = 0.0f;
    for (int d = 0; d < D; ++d) s = fmaf(qs[d], kv_load<KVT>(a.k_shared, row + d), s);
    s *= c;
    ss[t] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.0f;
  for (int t = tid; t < n; t += 256) {
    const float p = fast_exp2(ss[t] - mx);
    ss[t] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = sum;
  __syncthreads();
  sum = red[4] + red[5] + red[6] + red[7];
  for (int d = tid; d < D; d += 256) {
    const size_t vrow = vbase + (size_t)d * rd.Pp + wk.p0;
    float acc = 0.0f;
    for (int t = 0; t < n; ++t) acc = fmaf(ss[t], kv_load<KVT>(a.v_shared, vrow + t), acc);
    a.opart[(((size_t)wk.split * a.sumW + slot) * a.Hq + qh) * D + d] = acc * vscale / sum;
  }
  if (tid == 0) a.lpart[((size_t)wk.split * a.sumW + slot) * a.Hq + qh] = (mx + fast_log2(sum)) * kLn2;
}

}  // namespace

hipError_t launch_attn_shared_mfma(const AttnArgs& a, const ShWork* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  if (a.kv_dtype == GRW_FP8_E4M3)
    attn_shared_mfma_kernel<true><<<n_work, 256, 0, s>>>(a, work);
  else
    attn_shared_mfma_kernel<false><<<n_work, 256, 0, s>>>(a, work);
  return hipGetLastError();
}

hipError_t launch_attn_shared_split(const AttnArgs& a, const ShWork* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  static bool attr_set = false;   // the rings and P buffers need more than the default 64 KB of LDS
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)split::attn_shared_split_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, split::SMEM_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  split::attn_shared_split_kernel<<<n_work, split::NWAVES * 64, split::SMEM_BYTES, s>>>(a, work);
  return hipGetLastError();
}

hipError_t launch_attn_shared_valu(const AttnArgs& a, const ShWork* work, int n_work, hipStream_t s) {
  if (n_work <= 0) return hipSuccess;
  switch (a.kv_dtype) {
    case GRW_F32: attn_shared_valu_kernel<GRW_F32><<<n_work, 256, 0, s>>>(a, work); break;
    case GRW_BF16: attn_shared_valu_kernel<GRW_BF16><<<n_work, 256, 0, s>>>(a, work); break;
    default: attn_shared_valu_kernel<GRW_FP8_E4M3><<<n_work, 256, 0, s>>>(a, work); break;
  }
  return hipGetLastError();
}

}  // namespace grw
