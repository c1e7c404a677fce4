// a4: the log-sum-exp merge of a request's split partials, one (request, kv
// head) and one slab of output columns per workgroup.  A device function so
// that k_attn_merge and the drafter layer's combined scan + merge launch
// (ssd.hip) run the same code.
#pragma once

#include "common.h"
#include "kernels.h"

namespace hspec {

// LPO lanes (1 or 4) per (row, 4 output columns), in log2 units like the
// partials: lane q takes splits q, q+LPO, ..., loading U of them at a time
// (clamped indices, no data-dependent branches) and keeping a running
// maximum; with LPO = 4 the quad then combines its four (m, l, O) with two
// xor-shuffles.  A request with up to LPO*U splits costs one round of
// independent loads; LPO and U are sized to the largest split count at launch
// so few loads are clamped repeats and few lanes idle.
// (bx, by): the merge grid's block index (request * Hkv + kv head, column slab).
template <typename T, int D, int LPO, int U>
__device__ __forceinline__ void attn_merge_block(const AttnArgs& a, int bx, int by) {
  constexpr int OPB = 256 / LPO;  // outputs per block
  const int Hkv = a.Hkv;
  const int b = bx / Hkv, j = bx % Hkv;
  const int ctx = min(max(a.ctx_lens[b], 0), a.max_ctx);
  const int ns = max(1, (((ctx + 15) >> 4) + a.pps - 1) / a.pps);
  if (ns <= 1) return;
  const int rows = a.rows, G = a.G, K = a.K;
  const int idx = by * OPB + int(threadIdx.x) / LPO, q = int(threadIdx.x) % LPO;
  const bool live = idx < rows * (D / 4);  // whole quads agree
  const int row = min(idx / (D / 4), rows - 1), d4 = idx % (D / 4);
  const size_t stride = size_t(Hkv) * rows;  // partial rows between consecutive splits
  const size_t p0 = (size_t(b) * a.max_splits * Hkv + j) * rows + row;
  float M = -INFINITY, Ls = 0.f;
  float4 acc = make_float4(0, 0, 0, 0);
  for (int s0 = q; s0 < ns; s0 += LPO * U) {
    float2 ml[U];
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t pr = p0 + size_t(min(s0 + LPO * u, ns - 1)) * stride;
      ml[u] = *reinterpret_cast<const float2*>(a.part_ml + pr * 2);
      v[u] = reinterpret_cast<const float4*>(a.part_o + pr * D)[d4];
    }
    float mr = M;  // every split holds at least one token: its maximum is finite
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + LPO * u < ns) mr = fmaxf(mr, ml[u].x);
    const float sc = M == -INFINITY ? 0.f : fast_exp2(M - mr);
    acc.x *= sc; acc.y *= sc; acc.z *= sc; acc.w *= sc;
    Ls *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float f = s0 + LPO * u < ns ? fast_exp2(ml[u].x - mr) : 0.f;
      acc.x += f * v[u].x; acc.y += f * v[u].y; acc.z += f * v[u].z; acc.w += f * v[u].w;
      Ls += f * ml[u].y;
    }
    M = mr;
  }
  // combine the quad (a lane without splits has M = -inf, Ls = 0, acc = 0)
#pragma unroll
  for (int x = 1; x < LPO; x <<= 1) {
    const float Mo = __shfl_xor(M, x, 64), Lo = __shfl_xor(Ls, x, 64);
    const float ox = __shfl_xor(acc.x, x, 64), oy = __shfl_xor(acc.y, x, 64);
    const float oz = __shfl_xor(acc.z, x, 64), ow = __shfl_xor(acc.w, x, 64);
    const float Mn = fmaxf(M, Mo);
    const float f1 = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
    const float f2 = Mo == -INFINITY ? 0.f : fast_exp2(Mo - Mn);
    acc.x = acc.x * f1 + ox * f2; acc.y = acc.y * f1 + oy * f2;
    acc.z = acc.z * f1 + oz * f2; acc.w = acc.w * f1 + ow * f2;
    Ls = Ls * f1 + Lo * f2;
    M = Mn;
  }
  if (!live || q != 0) return;
  const float inv = 1.f / Ls;
  const int t = row / G, gg = row % G;
  T* o = static_cast<T*>(a.out) + ((size_t(b) * K + t) * a.Hq + j * G + gg) * D + d4 * 4;
  if constexpr (sizeof(T) == 2) {
    uint2 w;
    w.x = pack_bf16x2(acc.x * inv, acc.y * inv);
    w.y = pack_bf16x2(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2*>(o) = w;
  } else {
    *reinterpret_cast<float4*>(o) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
}

}  // namespace hspec
