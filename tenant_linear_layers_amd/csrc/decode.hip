// Decode-shaped BitDelta linear on gfx950 (M <= 64 tokens): one pass over
// W_base and the packed signs, both products on the matrix cores.
//
// Page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak", section
// "Sunum mimarisi": the fused kernel reads the base weights and the delta
// bits together and never writes W_eff = W_base + alpha*sign(Delta) to
// memory.  Here the product is split by linearity,
//     y[m, o] = sum_i x[m,i] W_base[o,i]  +  alpha_o * sum_i x[m,i] s[o,i],
// and both sums run as bf16 MFMA with float32 accumulation: the first takes
// W_base straight from memory as its B operand (no ALU work on the weights at
// all), the second takes +-1.0 in bf16 built from the sign bits, which is
// exact.  alpha is applied once per output, so no per-weight rounding of
// W_eff happens and the only roundings are the float32 accumulation and the
// final bf16 store.
//
// Work split: a workgroup owns 16 output rows; its NW waves split d_in into
// contiguous ranges of 128-element blocks and their partial accumulators are
// summed in LDS in a fixed order (deterministic).  Within a block, lane
// (n = lane%16, g = lane/16) holds 32 consecutive elements of row n (four
// 16-byte loads) and the 32 matching sign bits (one 4-byte load); the same
// lane holds the same 32 elements of token n of each 16-token tile.  MFMA
// 16x16x32 step q (0..3) uses the lane's elements 8q..8q+7 for both operands.
#include "common.h"
#include "internal.h"

namespace bd {
namespace {

// +-1.0 bf16 pairs for the lane's 32 elements from their sign bits
// (bit e = element e, 1 meaning +1).  Dword i pairs elements 2i (low half)
// and 2i+1 (high half), the same pairing as the bf16 data dwords.
// The negated bits are first spread so that the bits of elements 2i and
// 2i+1 sit 16 places apart (zl for i < 8, zh for i >= 8); one shift then
// puts both onto the two bf16 sign positions 15 and 31.
__device__ __forceinline__ void sign_pairs(uint32_t bits, uint32_t (&s)[16]) {
  const uint32_t nb = ~bits;
  const uint32_t zl = (nb & 0x00005555u) | ((nb << 15) & 0xFFFFAAAAu);
  const uint32_t zh = ((nb >> 16) & 0x00005555u) | ((nb >> 1) & 0xFFFFAAAAu);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s[i] = ((zl << (15 - 2 * i)) & 0x80008000u) | 0x3F803F80u;
    s[i + 8] = ((zh << (15 - 2 * i)) & 0x80008000u) | 0x3F803F80u;
  }
}

__device__ __forceinline__ u32x4 quad(const uint32_t (&s)[16], int q) {
  u32x4 v = {s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
  return v;
}

__device__ __forceinline__ u32x4 masked(u32x4 v, bool keep) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return keep ? v : z;
}

// Grouping of a mixed batch by variant, built once per workgroup in LDS.
// Tokens are ordered by variant id (stable); slot s of the sorted order holds
// token perm[s] of variant slotv[s] (-1 base only, -2 invalid id).  A "pair"
// is a maximal run of slots of one variant inside one 16-token tile.
struct Groups {
  int perm[kMaxSkinnyTokens];
  int slotv[kMaxSkinnyTokens];
  int pv[kMaxSkinnyTokens];
  int pt[kMaxSkinnyTokens];
  int plo[kMaxSkinnyTokens];
  int phi[kMaxSkinnyTokens];
  int key[kMaxSkinnyTokens];
  int dv[kMaxSkinnyTokens];   // distinct variants present, ascending
  int dp0[kMaxSkinnyTokens];  // first pair of each distinct variant
  int dp1[kMaxSkinnyTokens];  // one past its last pair
  int np;
  int nd;
};

__device__ void build_groups(Groups& G, const int32_t* ids, int M, int n_variants) {
  const int t = threadIdx.x;
  if (t < M) {
    const int v = ids[t];
    // order: variants 0..V-1, then base-only tokens, then invalid ids
    G.key[t] = (v >= 0 && v < n_variants) ? v : (v == -1 ? n_variants : n_variants + 1);
  }
  __syncthreads();
  if (t < M) {
    const int k = G.key[t];
    int rank = 0;
    for (int u = 0; u < M; ++u) {
      const int ku = G.key[u];
      rank += (ku < k || (ku == k && u < t)) ? 1 : 0;
    }
    G.perm[rank] = t;
    G.slotv[rank] = k < n_variants ? k : (k == n_variants ? -1 : -2);
  }
  __syncthreads();
  if (t < M) {
    const int v = G.slotv[t];
    const bool start = v >= 0 && (t % 16 == 0 || G.slotv[t - 1] != v);
    if (start) {
      int idx = 0;
      for (int u = 0; u < t; ++u) {
        const int vu = G.slotv[u];
        idx += (vu >= 0 && (u % 16 == 0 || G.slotv[u - 1] != vu)) ? 1 : 0;
      }
      int end = t + 1;
      while (end < M && end % 16 != 0 && G.slotv[end] == v) ++end;
      G.pv[idx] = v;
      G.pt[idx] = t / 16;
      G.plo[idx] = t % 16;
      G.phi[idx] = end - (t / 16) * 16;
    }
  }
  __syncthreads();
  if (t == 0) {
    int np = 0, nd = 0;
    for (int u = 0; u < M; ++u) {
      const int vu = G.slotv[u];
      if (vu >= 0 && (u % 16 == 0 || G.slotv[u - 1] != vu)) {
        if (nd == 0 || G.dv[nd - 1] != vu) {
          if (nd > 0) G.dp1[nd - 1] = np;
          G.dv[nd] = vu;
          G.dp0[nd] = np;
          ++nd;
        }
        ++np;
      }
    }
    if (nd > 0) G.dp1[nd - 1] = np;
    G.np = np;
    G.nd = nd;
  }
  __syncthreads();
}

template <int MT, int NW, int U, bool kMulti>
__global__ __launch_bounds__(NW * kWave) void linear_skinny_kernel(const SkinnyArgs a) {
  __shared__ float red[NW * MT * 2 * 4 * kWave];
  __shared__ Groups G;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int d_in = a.d_in;
  const int M = a.M;
  const int row = min(row0 + n, a.d_out - 1);

  if (kMulti) build_groups(G, a.ids, M, a.n_variants);

  const uint16_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int slot = min(16 * t + n, M - 1);
    const int tok = kMulti ? G.perm[slot] : slot;
    xrow[t] = a.x + (size_t)tok * d_in;
  }
  const uint16_t* wrow = a.w + (size_t)row * d_in;
  const size_t brow = (size_t)row * (d_in >> 5);

  f32x4 accw[MT], accs[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    accw[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    accs[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nblk = (d_in + 127) >> 7;
  const int b0 = (wv * nblk) / NW;
  const int b1 = ((wv + 1) * nblk) / NW;
  const int nd = kMulti ? G.nd : 0;

  // Groups of U blocks: every load of a group is issued before the first
  // MFMA that needs it, so each wave keeps U blocks of weights in flight.
  // Loads are never predicated (a lane-dependent load would force a wait on
  // the register it shares with the zero fill): a block past the wave's
  // range re-reads the last valid block and is skipped, and the lanes of a
  // final 64-wide block that fall past d_in re-read valid data whose x is
  // then zeroed.
  const bool half_tail = (d_in & 127) != 0;
  for (int b = b0; b < b1; b += U) {
    u32x4 wf[U][4];
    u32x4 xf[U][MT][4];
    uint32_t bits[U];
    size_t boff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int bu = min(b + u, b1 - 1);
      const int kc = min((bu << 7) + (g << 5), d_in - 32);
      boff[u] = brow + (kc >> 5);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wf[u][q] = ld128(wrow + kc + 8 * q);
#pragma unroll
        for (int t = 0; t < MT; ++t) xf[u][t][q] = ld128(xrow[t] + kc + 8 * q);
      }
      if (!kMulti) bits[u] = ld32(a.packed[0] + boff[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (half_tail && b + u == nblk - 1 && ((b + u) << 7) + (g << 5) >= d_in) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) xf[u][t][q] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (!kMulti) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b + u >= b1) continue;  // uniform
        uint32_t s[16];
        sign_pairs(bits[u], s);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            accw[t] = mfma16(xf[u][t][q], wf[u][q], accw[t]);
            accs[t] = mfma16(xf[u][t][q], quad(s, q), accs[t]);
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b + u >= b1) continue;  // uniform
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int t = 0; t < MT; ++t) accw[t] = mfma16(xf[u][t][q], wf[u][q], accw[t]);
      }
      // One distinct variant at a time; its sign words for the U blocks are
      // fetched while the previous variant's MFMAs run.
      uint32_t nxt[U];
      if (nd > 0) {
        const int v0 = __builtin_amdgcn_readfirstlane(G.dv[0]);
#pragma unroll
        for (int u = 0; u < U; ++u) nxt[u] = ld32(a.packed[v0] + boff[u]);
      }
      for (int d = 0; d < nd; ++d) {
        uint32_t cur[U];
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        if (d + 1 < nd) {
          const int vn = __builtin_amdgcn_readfirstlane(G.dv[d + 1]);
#pragma unroll
          for (int u = 0; u < U; ++u) nxt[u] = ld32(a.packed[vn] + boff[u]);
        }
        const int p0 = __builtin_amdgcn_readfirstlane(G.dp0[d]);
        const int p1 = __builtin_amdgcn_readfirstlane(G.dp1[d]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (b + u >= b1) continue;  // uniform
          uint32_t s[16];
          sign_pairs(cur[u], s);
          for (int p = p0; p < p1; ++p) {
            const int tp = __builtin_amdgcn_readfirstlane(G.pt[p]);
            const bool keep = n >= G.plo[p] && n < G.phi[p];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              if (t == tp) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  accs[t] = mfma16(masked(xf[u][t][q], keep), quad(s, q), accs[t]);
              }
            }
          }
        }
      }
    }
  }

  // Partial sums of the NW waves -> LDS, then a fixed-order sum per output.
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      red[(((wv * MT + t) * 2 + 0) * 4 + v) * kWave + lane] = accw[t][v];
      red[(((wv * MT + t) * 2 + 1) * 4 + v) * kWave + lane] = accs[t][v];
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < MT * 4 * kWave; idx += NW * kWave) {
    const int l = idx & (kWave - 1);
    const int v = (idx >> 6) & 3;
    const int t = idx >> 8;
    float sw = 0.f, ss = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sw += red[(((w * MT + t) * 2 + 0) * 4 + v) * kWave + l];
      ss += red[(((w * MT + t) * 2 + 1) * 4 + v) * kWave + l];
    }
    // MFMA 16x16 output layout: lane l holds rows 4*(l/16)+v of column l%16.
    const int slot = 16 * t + 4 * (l >> 4) + v;
    const int o = row0 + (l & 15);
    if (slot < M && o < a.d_out) {
      float yv;
      int m;
      if (!kMulti) {
        m = slot;
        const float al = a.per_row ? a.alpha[0][o] : a.alpha[0][0];
        yv = sw + al * ss;
      } else {
        m = G.perm[slot];
        const int vv = G.slotv[slot];
        if (vv >= 0) {
          const float* ap = a.alpha[vv];
          const float al = a.per_row ? ap[o] : ap[0];
          yv = sw + al * ss;
        } else if (vv == -1) {
          yv = sw;
        } else {
          yv = __builtin_nanf("");
        }
      }
      a.y[(size_t)m * a.d_out + o] = f32_to_bf16_bits(yv);
    }
  }
}

template <int MT, bool kMulti>
hipError_t launch_mt(const SkinnyArgs& a, hipStream_t stream) {
  constexpr int NW = 8;
  constexpr int U = MT >= 4 ? 1 : (kMulti ? 4 / (2 * MT) : 4 / MT);
  const dim3 grid((a.d_out + 15) / 16);
  hipLaunchKernelGGL((linear_skinny_kernel<MT, NW, U, kMulti>), grid, dim3(NW * kWave), 0, stream,
                     a);
  return hipGetLastError();
}

template <bool kMulti>
hipError_t launch_any(const SkinnyArgs& a, hipStream_t stream) {
  if (a.M <= 16) return launch_mt<1, kMulti>(a, stream);
  if (a.M <= 32) return launch_mt<2, kMulti>(a, stream);
  return launch_mt<4, kMulti>(a, stream);
}

}  // namespace

hipError_t launch_linear_skinny(const SkinnyArgs& a, hipStream_t stream) {
  return launch_any<false>(a, stream);
}

hipError_t launch_linear_multi(const SkinnyArgs& a, hipStream_t stream) {
  return launch_any<true>(a, stream);
}

}  // namespace bd
