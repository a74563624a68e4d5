// Unshared stage and merge of beam attention (xLLM generative-recommendation design doc,
// section 4.2.2 stages 2 and 3; section 4.2.1 for the token-granular decode KV).
//
// Unshared stage: NW wavefronts per beam slot, each for Hkv/NW of its kv heads.  A wave
// walks the beam's parent pointers (j_d = b, j_{e-1} = parent[e][j_e]) and attends to the
// d + 1 decode tokens of its ancestry directly where they were written — no block copy, no
// reorder of the decode KV after selection.  Each lane holds E = Hkv*D/(64*NW) contiguous
// elements of the token's K and V rows (one kv head spans D/E lanes) and the matching
// elements of the beam's G query heads of that kv head; the next parent pointer is loaded
// together with the current token's K/V so the pointer chase overlaps the KV reads.  More
// waves per slot give a narrow batch more loads in flight.
//
// Merge: per (slot, query head) the partials i (the shared stage's splits and the
// unshared stage) combine as lse = log sum_i exp(lse_i), o = sum_i exp(lse_i - lse) o_i
// (online-softmax merge).  Dead slots (negative parent pointer at this depth) get zeros.
// The merge runs either as its own kernel over partials in the workspace, or fused into
// the unshared kernel's epilogue (the default path), where the unshared partial never
// leaves registers.
#include "device_common.h"
#include "grw_internal.h"

namespace grw {

namespace {

template <int KVT, int E>
__device__ __forceinline__ void load_row(const void* base, size_t off, float (&x)[E]) {
  if constexpr (KVT == GRW_F32) {
    const float* p = (const float*)base + off;
#pragma unroll
    for (int i = 0; i < E; i += 2) {
      floatx2 v = *(const floatx2*)(p + i);
      x[i] = v.x;
      x[i + 1] = v.y;
    }
  } else if constexpr (KVT == GRW_BF16) {
    const uint16_t* p = (const uint16_t*)base + off;
    if constexpr (E >= 8) {
#pragma unroll
      for (int i = 0; i < E; i += 8) {
        u32x4 w = *(const u32x4*)(p + i);
        x[i + 0] = __uint_as_float(w.x << 16); x[i + 1] = __uint_as_float(w.x & 0xFFFF0000u);
        x[i + 2] = __uint_as_float(w.y << 16); x[i + 3] = __uint_as_float(w.y & 0xFFFF0000u);
        x[i + 4] = __uint_as_float(w.z << 16); x[i + 5] = __uint_as_float(w.z & 0xFFFF0000u);
        x[i + 6] = __uint_as_float(w.w << 16); x[i + 7] = __uint_as_float(w.w & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < E; i += 2) {
        uint32_t w = *(const uint32_t*)(p + i);
        x[i] = __uint_as_float(w << 16);
        x[i + 1] = __uint_as_float(w & 0xFFFF0000u);
      }
    }
  } else {
    const uint8_t* p = (const uint8_t*)base + off;
    if constexpr (E >= 4) {
#pragma unroll
      for (int i = 0; i < E; i += 4) {
        const uint32_t w = *(const uint32_t*)(p + i);
        floatx2 lo = fp8x2_to_f32<false>(w), hi = fp8x2_to_f32<true>(w);
        x[i] = lo.x; x[i + 1] = lo.y; x[i + 2] = hi.x; x[i + 3] = hi.y;
      }
    } else {
      const uint32_t w = *(const uint16_t*)p;
      floatx2 lo = fp8x2_to_f32<false>(w);
      x[0] = lo.x; x[1] = lo.y;
    }
  }
}

// FUSE: merge the unshared partial with the shared stage's partials in the epilogue and
// write `out` directly (dead slots write zeros); otherwise write the unshared partial.
template <int KVT, int E, int G, int NW, bool FUSE>
__global__ __launch_bounds__(256) void attn_unshared_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int slot = gw / NW;
  if (slot >= a.sumW) return;
  const int sumW = a.sumW, D = a.D, Hq = a.Hq;
  const int LPH = D / E;                 // lanes per kv head
  const int hl = lane / LPH;             // this lane's kv head within the wave's share
  const int hk = (gw - slot * NW) * (64 / LPH) + hl;   // this lane's kv head
  const int d0 = (lane - hl * LPH) * E;  // first head-dim element of this lane
  const int step = a.step;

  const int par = a.parent_idx[(size_t)step * sumW + slot];
  if (par < 0) {                         // dead slot: zero output
    if constexpr (FUSE) {
#pragma unroll
      for (int jj = 0; jj < G; ++jj) {
        float* dst = a.out + ((size_t)slot * Hq + hk * G + jj) * D + d0;
#pragma unroll
        for (int i = 0; i < E; ++i) dst[i] = 0.0f;
      }
    }
    return;
  }
  const ReqDesc rd = a.req[a.slot_req[slot]];
  const int Wr = rd.W, boff = rd.boff;

  float q[G][E];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const size_t qi = ((size_t)slot * Hq + hk * G + j) * D + d0;
    if (a.q_dtype == GRW_F32) {
#pragma unroll
      for (int i = 0; i < E; ++i) q[j][i] = ((const float*)a.q)[qi + i];
    } else {
      load_row<GRW_BF16, E>(a.q, qi, q[j]);
    }
  }
  float c = rsqrtf((float)D) * kLog2e;
  float vscale = 1.0f;
  if constexpr (KVT == GRW_FP8_E4M3) {
    c *= a.k_scale[hk];
    vscale = a.v_scale[hk];
  }

  float m[G], l[G], o[G][E];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) o[j][i] = 0.0f;
  }

  const size_t tok = (size_t)a.Hkv * D;        // elements per decode token row
  int j = slot - boff;                          // request-local slot at depth e
  bool bad = false;
  for (int e = step; e >= 0; --e) {
    const size_t off = ((size_t)e * sumW + boff + j) * tok + (size_t)hk * D + d0;
    float kx[E], vx[E];
    load_row<KVT, E>(a.k_unshared, off, kx);
    load_row<KVT, E>(a.v_unshared, off, vx);
    int nj = 0;
    if (e > 0) nj = a.parent_idx[(size_t)e * sumW + boff + j];
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < E; ++i) s = fmaf(q[jj][i], kx[i], s);
      // sum over the head's LPH lanes (xor distances 1, 2, ... below LPH; LPH is wave-uniform)
      if (LPH > 1) s += lane_xor<1>(s);
      if (LPH > 2) s += lane_xor<2>(s);
      if (LPH > 4) s += lane_xor<4>(s);
      if (LPH > 8) s += lane_xor<8>(s);
      if (LPH > 16) s += lane_xor<16>(s);
      if (LPH > 32) s += lane_xor<32>(s);
      s *= c;
      const float mn = fmaxf(m[jj], s);
      const float alpha = fast_exp2(m[jj] - mn);
      const float p = fast_exp2(s - mn);
      l[jj] = fmaf(l[jj], alpha, p);
#pragma unroll
      for (int i = 0; i < E; ++i) o[jj][i] = fmaf(o[jj][i], alpha, p * vx[i]);
      m[jj] = mn;
    }
    if (e > 0) {
      if (nj < 0 || nj >= Wr) { bad = true; break; }
      j = nj;
    }
  }
  if (bad) {
    if (lane == 0) atomicOr(a.flags, (int)GRW_FLAG_BAD_PARENT);
    return;
  }
  if constexpr (!FUSE) {
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
      const float inv = vscale / l[jj];
      float* dst = a.ou + ((size_t)slot * Hq + hk * G + jj) * D + d0;
#pragma unroll
      for (int i = 0; i < E; ++i) dst[i] = o[jj][i] * inv;
      if (lane == hl * LPH) a.lu[(size_t)slot * Hq + hk * G + jj] = (m[jj] + fast_log2(l[jj])) * kLn2;
    }
  } else {
    // online-softmax merge with the shared partials, in log2 units:
    // weight of a partial = 2^(lse2_i - M), unshared weight = l * 2^(m - M) on the raw sums
    const int ns = rd.nsplit;
    const size_t plane = (size_t)sumW * Hq;
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
      const size_t row = (size_t)slot * Hq + hk * G + jj;
      float M = m[jj] + fast_log2(l[jj]);          // log2 of the unshared partial's mass
      for (int i = 0; i < ns; ++i) M = fmaxf(M, a.lpart[i * plane + row] * kLog2e);
      const float wu = fast_exp2(m[jj] - M) * vscale;   // multiplies the raw sum o
      float wsum = l[jj] * fast_exp2(m[jj] - M);
      float acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = o[jj][e] * wu;
      for (int i = 0; i < ns; ++i) {
        const float w = fast_exp2(a.lpart[i * plane + row] * kLog2e - M);
        wsum += w;
        const float* src = a.opart + (i * plane + row) * D + d0;
        if constexpr (E % 4 == 0) {
#pragma unroll
          for (int e = 0; e < E; e += 4) {
            const floatx4 v = *(const floatx4*)(src + e);
            acc[e] = fmaf(v.x, w, acc[e]);
            acc[e + 1] = fmaf(v.y, w, acc[e + 1]);
            acc[e + 2] = fmaf(v.z, w, acc[e + 2]);
            acc[e + 3] = fmaf(v.w, w, acc[e + 3]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] = fmaf(src[e], w, acc[e]);
        }
      }
      const float inv = 1.0f / wsum;
      float* dst = a.out + row * D + d0;
      if constexpr (E % 4 == 0) {
#pragma unroll
        for (int e = 0; e < E; e += 4)
          *(floatx4*)(dst + e) = floatx4{acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) dst[e] = acc[e] * inv;
      }
    }
  }
}

// one thread per (slot, query head, 4 head-dim elements)
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int D4 = a.D >> 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.sumW * a.Hq * D4;
  if (idx >= total) return;
  const int slot = (int)(idx / ((int64_t)a.Hq * D4));
  const int rem = (int)(idx - (int64_t)slot * a.Hq * D4);
  const int qh = rem / D4, d4 = rem - qh * D4;
  floatx4* dst = (floatx4*)(a.out + ((size_t)slot * a.Hq + qh) * a.D) + d4;
  if (a.parent_idx[(size_t)a.step * a.sumW + slot] < 0) {
    *dst = floatx4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  const int ns = a.req[a.slot_req[slot]].nsplit;
  const size_t row = (size_t)slot * a.Hq + qh;
  const size_t plane = (size_t)a.sumW * a.Hq;
  const float lu = a.lu[row];
  float M = lu;
  for (int i = 0; i < ns; ++i) M = fmaxf(M, a.lpart[i * plane + row]);
  float wsum = fast_exp2((lu - M) * kLog2e);
  floatx4 acc = ((const floatx4*)(a.ou + row * a.D))[d4] * wsum;
  for (int i = 0; i < ns; ++i) {
    const float w = fast_exp2((a.lpart[i * plane + row] - M) * kLog2e);
    acc += ((const floatx4*)(a.opart + (i * plane + row) * a.D))[d4] * w;
    wsum += w;
  }
  *dst = acc * (1.0f / wsum);
}

template <int KVT, int E, int NW, bool FUSE>
hipError_t launch_unshared_g(const AttnArgs& a, hipStream_t s) {
  const int blocks = (int)(((int64_t)a.sumW * NW + 3) / 4);
  switch (a.g) {
    case 1: attn_unshared_kernel<KVT, E, 1, NW, FUSE><<<blocks, 256, 0, s>>>(a); break;
    case 2: attn_unshared_kernel<KVT, E, 2, NW, FUSE><<<blocks, 256, 0, s>>>(a); break;
    default: attn_unshared_kernel<KVT, E, 4, NW, FUSE><<<blocks, 256, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

// Waves per slot: rows of 16 elements per lane (Hkv*D = 1024) go to two waves of 8 each,
// which doubles the loads in flight per CU (one wave per slot leaves 2048 slots at two
// waves per SIMD).
inline int unshared_waves_per_slot(const AttnArgs& a) { return (a.Hkv * a.D) / 64 == 16 ? 2 : 1; }

template <int KVT, bool FUSE>
hipError_t launch_unshared_e(const AttnArgs& a, hipStream_t s) {
  if (unshared_waves_per_slot(a) == 2) return launch_unshared_g<KVT, 8, 2, FUSE>(a, s);
  switch ((a.Hkv * a.D) / 64) {
    case 2: return launch_unshared_g<KVT, 2, 1, FUSE>(a, s);
    case 4: return launch_unshared_g<KVT, 4, 1, FUSE>(a, s);
    case 8: return launch_unshared_g<KVT, 8, 1, FUSE>(a, s);
    default: return launch_unshared_g<KVT, 16, 1, FUSE>(a, s);
  }
}

template <bool FUSE>
hipError_t launch_unshared_t(const AttnArgs& a, hipStream_t s) {
  if (a.sumW == 0) return hipSuccess;
  switch (a.kv_dtype) {
    case GRW_F32: return launch_unshared_e<GRW_F32, FUSE>(a, s);
    case GRW_BF16: return launch_unshared_e<GRW_BF16, FUSE>(a, s);
    default: return launch_unshared_e<GRW_FP8_E4M3, FUSE>(a, s);
  }
}

}  // namespace

hipError_t launch_attn_unshared(const AttnArgs& a, hipStream_t s) { return launch_unshared_t<false>(a, s); }

hipError_t launch_attn_unshared_merge(const AttnArgs& a, hipStream_t s) { return launch_unshared_t<true>(a, s); }

hipError_t launch_attn_merge(const AttnArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.sumW * a.Hq * (a.D / 4);
  if (total == 0) return hipSuccess;
  attn_merge_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace grw
