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
// Work split: a workgroup owns 16 output rows; its NW waves take the
// 128-element blocks of d_in round-robin (block b -> wave b % NW), so at any
// time they work on NW consecutive blocks of the same rows and together
// consume whole cache lines of weights and of sign words.  Their partial
// accumulators are summed in LDS in a fixed order (deterministic).  Within a
// block, lane (n = lane%16, g = lane/16) holds 32 consecutive elements of row
// n (four 16-byte loads) and the 32 matching sign bits (one 4-byte load); the
// same lane holds the same 32 elements of token n of each 16-token tile.
// MFMA 16x16x32 step q (0..3) uses the lane's elements 8q..8q+7 for both
// operands.
//
// Loads are never predicated: a lane-dependent load compiles to a masked
// branch whose fill of the same register forces a wait on every load.  A
// block past a wave's range re-reads the wave's last block and is skipped;
// lanes of a final 64-wide block that fall past d_in re-read valid data whose
// x is then zeroed.
#include "common.h"
#include "internal.h"

namespace bd {
namespace {

// +-1.0 bf16 pairs for the lane's 32 elements from their sign bits
// (bit e = element e, 1 meaning +1).  Dword i pairs elements 2i (low half)
// and 2i+1 (high half), the same pairing as the bf16 data dwords.  The
// negated bits are first spread so that the bits of elements 2i and 2i+1 sit
// 16 places apart (zl for i < 8, zh for i >= 8); one shift then puts both
// onto the two bf16 sign positions 15 and 31, and one bitop3 keeps them and
// adds the exponent and mantissa of 1.0.
__device__ __forceinline__ void sign_pairs(uint32_t bits, uint32_t (&s)[16]) {
  // bitop3 table 0x1B: (~a & c) | (~b & ~c), a bit-select of the negated
  // inputs; table 0xEA: (a & b) | c.
  const uint32_t zl = __builtin_amdgcn_bitop3_b32(bits, bits << 15, 0x00005555u, 0x1B);
  const uint32_t zh = __builtin_amdgcn_bitop3_b32(bits >> 16, bits >> 1, 0x00005555u, 0x1B);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s[i] = __builtin_amdgcn_bitop3_b32(zl << (15 - 2 * i), 0x80008000u, 0x3F803F80u, 0xEA);
    s[i + 8] = __builtin_amdgcn_bitop3_b32(zh << (15 - 2 * i), 0x80008000u, 0x3F803F80u, 0xEA);
  }
}

__device__ __forceinline__ u32x4 quad(const uint32_t (&s)[16], int q) {
  u32x4 v = {s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
  return v;
}

// Number of a wave's blocks when NW waves take nblk blocks round-robin.
__device__ __forceinline__ int blocks_of_wave(int wv, int nblk, int NW) {
  return wv < nblk ? (nblk - 1 - wv) / NW + 1 : 0;
}

// Sum the NW waves' partial accumulators (LDS, fixed order) and store y.
// out(slot, o, sw, ss, m) returns the output value and sets its token m.
template <int MT, int NW, class Out>
__device__ __forceinline__ void reduce_and_store(float* red, const f32x4 (&accw)[MT],
                                                 const f32x4 (&accs)[MT], int row0, int M,
                                                 int d_out, uint16_t* y, Out out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
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
    if (slot < M && o < d_out) {
      int m;
      const float yv = out(slot, o, sw, ss, m);
      y[(size_t)m * d_out + o] = f32_to_bf16_bits(yv);
    }
  }
}

// ---------------------------------------------------------------- one variant
template <int MT, int NW, int U>
__global__ __launch_bounds__(NW * kWave) void linear_decode_kernel(const SkinnyArgs a) {
  __shared__ float red[NW * MT * 2 * 4 * kWave];

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int d_in = a.d_in;
  const int M = a.M;
  const int row = min(row0 + n, a.d_out - 1);

  const uint16_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xrow[t] = a.x + (size_t)min(16 * t + n, M - 1) * d_in;
  const uint16_t* wrow = a.w + (size_t)row * d_in;
  const uint32_t* brow = a.packed[0] + (size_t)row * (d_in >> 5);

  f32x4 accw[MT], accs[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    accw[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    accs[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nblk = (d_in + 127) >> 7;
  const int nmine = blocks_of_wave(wv, nblk, NW);
  const bool half_tail = (d_in & 127) != 0;
  // Groups of U blocks: every load of a group is issued before the first
  // MFMA that needs it, so each wave keeps U blocks of weights in flight.
  for (int i = 0; i < nmine; i += U) {
    u32x4 wf[U][4];
    u32x4 xf[U][MT][4];
    uint32_t bits[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int bu = wv + NW * min(i + u, nmine - 1);
      const int kc = min((bu << 7) + (g << 5), d_in - 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wf[u][q] = ld128(wrow + kc + 8 * q);
#pragma unroll
        for (int t = 0; t < MT; ++t) xf[u][t][q] = ld128(xrow[t] + kc + 8 * q);
      }
      bits[u] = ld32(brow + (kc >> 5));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i + u >= nmine) continue;  // uniform
      const int bu = wv + NW * (i + u);
      if (half_tail && bu == nblk - 1 && (bu << 7) + (g << 5) >= d_in) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) xf[u][t][q] = u32x4{0u, 0u, 0u, 0u};
      }
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
  }

  const float* alpha = a.alpha[0];
  const int per_row = a.per_row;
  reduce_and_store<MT, NW>(red, accw, accs, row0, M, a.d_out, a.y,
                           [&](int slot, int o, float sw, float ss, int& m) {
                             m = slot;
                             return sw + (per_row ? alpha[o] : alpha[0]) * ss;
                           });
}

// ---------------------------------------------------------------- mixed batch
// Grouping of a mixed batch by variant, built once per workgroup in LDS.
// Tokens are ordered by variant id (stable); slot s of the sorted order holds
// token perm[s] of variant slotv[s] (-1 base only, -2 invalid id).  A "pair"
// is a maximal run of slots of one variant inside one 16-token tile; dv[]
// lists the distinct variants present and [dp0, dp1) their pairs.
struct Groups {
  int perm[kMaxSkinnyTokens];
  int slotv[kMaxSkinnyTokens];
  int pt[kMaxSkinnyTokens];
  int plo[kMaxSkinnyTokens];
  int phi[kMaxSkinnyTokens];
  int key[kMaxSkinnyTokens];
  int dv[kMaxSkinnyTokens];
  int dp0[kMaxSkinnyTokens];
  int dp1[kMaxSkinnyTokens];
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

// The base product runs once for all tokens; the sign product once per
// distinct variant present, with the x tile masked to that variant's tokens.
// Each wave stages its x block in LDS next to a zero row: a variant's masked
// tile is read by choosing, per lane, its token row or the zero row (one
// address select instead of a select per register).  The distinct variants
// are taken one at a time, the next one's sign words already requested.
//
// RT row tiles share a workgroup: its NW waves are RT row tiles x NW/RT
// K-lanes, and the RT waves of one K-lane work on the same block at the same
// time, so their x loads are the same addresses and all but one hit in L1.
// With M = 32 the x bytes of a block are twice its weight bytes, so this
// cuts the L2 traffic of the kernel by about a third for RT = 2.
template <int MT, int NW, int RT>
__global__ __launch_bounds__(NW * kWave) void linear_multi_kernel(const SkinnyArgs a) {
  constexpr int KL = NW / RT;                  // K-lanes (waves per row tile)
  constexpr int kRedBytes = NW * MT * 2 * 4 * kWave * 4;
  constexpr int kXRow = 128 + 8;               // bf16 per staged row (padded)
  constexpr int kXRows = MT * 16 + 1;          // token rows + zero row
  constexpr int kXWave = kXRows * kXRow;       // bf16 per wave
  constexpr int kXBytes = NW * kXWave * 2;
  __shared__ __attribute__((aligned(16))) char smem[kRedBytes > kXBytes ? kRedBytes : kXBytes];
  __shared__ Groups G;

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int rt = wv % RT;
  const int kl = wv / RT;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int row0 = (blockIdx.x * RT + rt) * 16;
  const int d_in = a.d_in;
  const int M = a.M;
  const int row = min(row0 + n, a.d_out - 1);
  uint16_t* xst = reinterpret_cast<uint16_t*>(smem) + wv * kXWave;

  build_groups(G, a.ids, M, a.n_variants);
  for (int e = lane; e < kXRow / 2; e += kWave)
    reinterpret_cast<uint32_t*>(xst + MT * 16 * kXRow)[e] = 0u;

  const uint16_t* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xrow[t] = a.x + (size_t)G.perm[min(16 * t + n, M - 1)] * d_in;
  const uint16_t* wrow = a.w + (size_t)row * d_in;
  const size_t brow = (size_t)row * (d_in >> 5);

  f32x4 accw[MT], accs[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    accw[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    accs[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nblk = (d_in + 127) >> 7;
  const int nmine = blocks_of_wave(kl, nblk, KL);
  const bool half_tail = (d_in & 127) != 0;
  const int nd = G.nd;

  for (int i = 0; i < nmine; ++i) {
    const int bu = kl + KL * i;
    const int kc = min((bu << 7) + (g << 5), d_in - 32);
    u32x4 wf[4];
    u32x4 xf[MT][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wf[q] = ld128(wrow + kc + 8 * q);
#pragma unroll
      for (int t = 0; t < MT; ++t) xf[t][q] = ld128(xrow[t] + kc + 8 * q);
    }
    // first variant's sign words go out with the block's weights
    uint32_t nxt = 0u;
    if (nd > 0) {
      const int v0 = __builtin_amdgcn_readfirstlane(G.dv[0]);
      nxt = ld32(a.packed[v0] + brow + (kc >> 5));
    }
    if (half_tail && bu == nblk - 1 && (bu << 7) + (g << 5) >= d_in) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) xf[t][q] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4*>(xst + (16 * t + n) * kXRow + 32 * g + 8 * q) = xf[t][q];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < MT; ++t) accw[t] = mfma16(xf[t][q], wf[q], accw[t]);

    for (int d = 0; d < nd; ++d) {
      const uint32_t cur = nxt;
      if (d + 1 < nd) {
        const int vn = __builtin_amdgcn_readfirstlane(G.dv[d + 1]);
        nxt = ld32(a.packed[vn] + brow + (kc >> 5));
      }
      const int p0 = __builtin_amdgcn_readfirstlane(G.dp0[d]);
      const int p1 = __builtin_amdgcn_readfirstlane(G.dp1[d]);
      uint32_t s[16];
      sign_pairs(cur, s);
      for (int p = p0; p < p1; ++p) {
        const int tp = __builtin_amdgcn_readfirstlane(G.pt[p]);
        const int lo = __builtin_amdgcn_readfirstlane(G.plo[p]);
        const int hi = __builtin_amdgcn_readfirstlane(G.phi[p]);
        const bool keep = (unsigned)(n - lo) < (unsigned)(hi - lo);
        const uint16_t* src = xst + (keep ? 16 * tp + n : MT * 16) * kXRow + 32 * g;
        u32x4 xm[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) xm[q] = *reinterpret_cast<const u32x4*>(src + 8 * q);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t == tp) {
#pragma unroll
            for (int q = 0; q < 4; ++q) accs[t] = mfma16(xm[q], quad(s, q), accs[t]);
          }
        }
      }
    }
  }

  // The LDS region may still hold other waves' staged x: barrier first.
  __syncthreads();
  // Partial sums: wave (rt, kl) -> its row tile's K-lane kl.
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      red[(((wv * MT + t) * 2 + 0) * 4 + v) * kWave + lane] = accw[t][v];
      red[(((wv * MT + t) * 2 + 1) * 4 + v) * kWave + lane] = accs[t][v];
    }
  }
  __syncthreads();
  const int per_row = a.per_row;
  for (int idx = threadIdx.x; idx < RT * MT * 4 * kWave; idx += NW * kWave) {
    const int l = idx & (kWave - 1);
    const int v = (idx >> 6) & 3;
    const int t = (idx >> 8) % MT;
    const int r = (idx >> 8) / MT;
    float sw = 0.f, ss = 0.f;
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      const int w = k * RT + r;
      sw += red[(((w * MT + t) * 2 + 0) * 4 + v) * kWave + l];
      ss += red[(((w * MT + t) * 2 + 1) * 4 + v) * kWave + l];
    }
    // MFMA 16x16 output layout: lane l holds rows 4*(l/16)+v of column l%16.
    const int slot = 16 * t + 4 * (l >> 4) + v;
    const int o = (blockIdx.x * RT + r) * 16 + (l & 15);
    if (slot < M && o < a.d_out) {
      const int m = G.perm[slot];
      const int vv = G.slotv[slot];
      float yv;
      if (vv >= 0) {
        const float* ap = a.alpha[vv];
        yv = sw + (per_row ? ap[o] : ap[0]) * ss;
      } else {
        yv = vv == -1 ? sw : __builtin_nanf("");
      }
      a.y[(size_t)m * a.d_out + o] = f32_to_bf16_bits(yv);
    }
  }
}

// ---------------------------------------------------------------- launchers
constexpr int kNW = 8;

template <int MT>
hipError_t launch_decode(const SkinnyArgs& a, hipStream_t stream) {
  constexpr int U = MT >= 4 ? 1 : 4 / MT;
  hipLaunchKernelGGL((linear_decode_kernel<MT, kNW, U>), dim3((a.d_out + 15) / 16),
                     dim3(kNW * kWave), 0, stream, a);
  return hipGetLastError();
}

template <int MT, int RT>
hipError_t launch_multi_rt(const SkinnyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((linear_multi_kernel<MT, kNW, RT>), dim3((a.d_out + 16 * RT - 1) / (16 * RT)),
                     dim3(kNW * kWave), 0, stream, a);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_multi(const SkinnyArgs& a, hipStream_t stream) {
  // One row tile per workgroup: measured on the 70B-shaped gate matrix
  // (M = 32, 14 variants), two row tiles sharing x through L1 were 6% slower.
  return launch_multi_rt<MT, 1>(a, stream);
}

}  // namespace

hipError_t launch_linear_skinny(const SkinnyArgs& a, hipStream_t stream) {
  if (a.M <= 16) return launch_decode<1>(a, stream);
  if (a.M <= 32) return launch_decode<2>(a, stream);
  return launch_decode<4>(a, stream);
}

hipError_t launch_linear_multi(const SkinnyArgs& a, hipStream_t stream) {
  if (a.M <= 16) return launch_multi<1>(a, stream);
  if (a.M <= 32) return launch_multi<2>(a, stream);
  return launch_multi<4>(a, stream);
}

}  // namespace bd
