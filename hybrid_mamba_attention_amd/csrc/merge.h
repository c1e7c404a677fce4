// a4: the log-sum-exp merge of a request's pieces (the partials its work
// ranges left), one (request, kv head) and one slab of output columns per
// workgroup.  A device function so that k_attn_merge and the drafter layer's
// combined scan + merge launch (ssd.hip) run the same code.
#pragma once

#include "common.h"
#include "kernels.h"

namespace hspec {

// LPO lanes (1 or 4) per (row, 4 output columns), in log2 units like the
// partials: lane q takes pieces q, q+LPO, ..., loading up to U of them at a
// time (clamped indices, no data-dependent branches inside a round) and
// keeping a running maximum; with LPO = 4 the quad then combines its four
// (m, l, O) with two xor-shuffles.  LPO and U are sized at launch to the
// most pieces a request can have; the loads per round follow the request's
// own count, so a request of up to LPO*U pieces costs one round of
// independent loads with few clamped repeats.
// The request's pieces come from the work plan the attention grid wrote:
// piece i sits in slot 2*(w_first + i) (+1 for the first piece when the
// request starts after its first range's first granule).
// (bx, by): the merge grid's block index (request * Hkv + kv head, column slab).
template <typename T, int D, int LPO, int U>
__device__ __forceinline__ void attn_merge_block(const AttnArgs& a, int bx, int by) {
  constexpr int OPB = 256 / LPO;  // outputs per block
  const int Hkv = a.Hkv, C = a.C;
  const int b = bx / Hkv, j = bx % Hkv;
  const int32_t* plan = a.plan;
  const int ns = plan[4 + 2 * C + b];
  if (ns <= 1) return;   // finished by its one range
  const int wf = plan[4 + C + b];
  const int k0 = plan[4 + 3 * C + wf] < plan[4 + b] ? 1 : 0;
  const int rows = a.rows, G = a.G, K = a.K;
  const int idx = by * OPB + int(threadIdx.x) / LPO, q = int(threadIdx.x) % LPO;
  const bool live = idx < rows * (D / 4);  // whole quads agree
  const int row = min(idx / (D / 4), rows - 1), d4 = idx % (D / 4);
  auto prow = [&](int i) -> size_t {     // partial row of piece i
    const int slot = 2 * (wf + i) + (i == 0 ? k0 : 0);
    return (size_t(slot) * Hkv + j) * rows + row;
  };
  float M = -INFINITY, Ls = 0.f;
  float4 acc = make_float4(0, 0, 0, 0);
  // Rounds of UU loads per lane, all issued before the first use.
  auto rounds = [&](auto UC) __attribute__((always_inline)) {
    constexpr int UU = decltype(UC)::value;
    for (int s0 = q; s0 < ns; s0 += LPO * UU) {
      float2 ml[UU];
      float4 v[UU];
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        const size_t pr = prow(min(s0 + LPO * u, ns - 1));
        ml[u] = *reinterpret_cast<const float2*>(a.part_ml + pr * 2);
        if constexpr (sizeof(T) == 2) {   // four bf16 of the piece's normalised output
          const uint2 x = reinterpret_cast<const uint2*>(static_cast<const T*>(a.part_o) + pr * D)[d4];
          v[u] = make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                             __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
        } else {
          v[u] = reinterpret_cast<const float4*>(static_cast<const float*>(a.part_o) + pr * D)[d4];
        }
      }
      // A piece's maximum is -inf when the block-causal mask hides all its
      // keys from this row (a piece of block keys only); such a piece weighs
      // 0.  The request's first piece always holds a key every row sees (its
      // context or block key 0), so the total weight is positive.
      float mr = M;
#pragma unroll
      for (int u = 0; u < UU; ++u)
        if (s0 + LPO * u < ns) mr = fmaxf(mr, ml[u].x);
      const float sc = M == -INFINITY ? 0.f : fast_exp2(M - mr);
      acc.x *= sc; acc.y *= sc; acc.z *= sc; acc.w *= sc;
      Ls *= sc;
#pragma unroll
      for (int u = 0; u < UU; ++u) {
        // a piece weighs l e^(m - M): its output is stored divided by its l
        const float f = (s0 + LPO * u < ns && ml[u].x != -INFINITY) ? fast_exp2(ml[u].x - mr) * ml[u].y : 0.f;
        acc.x += f * v[u].x; acc.y += f * v[u].y; acc.z += f * v[u].z; acc.w += f * v[u].w;
        Ls += f;
      }
      M = mr;
    }
  };
  // Loads per lane and round by the request's own piece count (uniform over
  // the workgroup): sized by the most pieces any request could have, a
  // request of two pieces would issue up to LPO * U clamped repeats per
  // output, which dominated the merge when ranges cut most requests in two.
  const int per_lane = (ns + LPO - 1) / LPO;
  if (per_lane <= 1 || U == 1) rounds(std::integral_constant<int, 1>{});
  else if (per_lane <= 2 || U == 2) rounds(std::integral_constant<int, 2>{});
  else if (per_lane <= 4 || U == 4) rounds(std::integral_constant<int, 4>{});
  else rounds(std::integral_constant<int, U>{});
  // combine the quad (a lane without pieces has M = -inf, Ls = 0, acc = 0)
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
