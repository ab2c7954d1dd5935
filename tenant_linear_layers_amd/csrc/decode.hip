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
// token perm[s] of variant slotv[s] (-1 base only, -2 invalid id).  The slots
// of one variant form a run; a "window" is a piece of at most 16 slots of a
// run (runs are cut every 16 slots from their start): window w covers slots
// ws0[w] .. ws0[w] + wlen[w] - 1, all of variant wvar[w].
struct Groups {
  int perm[kMaxSkinnyTokens];
  int slotv[kMaxSkinnyTokens];
  int key[kMaxSkinnyTokens];
  int wvar[kMaxSkinnyTokens];
  int ws0[kMaxSkinnyTokens];
  int wlen[kMaxSkinnyTokens];
  int nwin;
};

__device__ void build_groups(Groups& G, const int32_t* ids, int M, int n_variants) {
  const int t = threadIdx.x;
  if (t < M) {
    const int v = ids[t];
    // order: variants 0..V-1, then base-only tokens, then invalid ids
    G.key[t] = (v >= 0 && v < n_variants) ? v : (v == -1 ? n_variants : n_variants + 1);
  }
  __syncthreads();
  int k = 0;
  if (t < M) {
    k = G.key[t];
    int rank = 0;
    for (int u = 0; u < M; ++u) {
      const int ku = G.key[u];
      rank += (ku < k || (ku == k && u < t)) ? 1 : 0;
    }
    G.perm[rank] = t;
    G.slotv[rank] = k < n_variants ? k : (k == n_variants ? -1 : -2);
  }
  __syncthreads();
  // window starts: slots of a variant whose offset in the variant's run is a
  // multiple of 16 (key[] is free again and marks them)
  if (t < M) {
    const int v = G.slotv[t];
    int rs = t;
    while (rs > 0 && G.slotv[rs - 1] == v) --rs;
    G.key[t] = (v >= 0 && (t - rs) % 16 == 0) ? 1 : 0;
  }
  __syncthreads();
  if (t < M && G.key[t]) {
    const int v = G.slotv[t];
    int idx = 0;
    for (int u = 0; u < t; ++u) idx += G.key[u];
    int len = 1;
    while (t + len < M && len < 16 && G.slotv[t + len] == v) ++len;
    G.wvar[idx] = v;
    G.ws0[idx] = t;
    G.wlen[idx] = len;
  }
  if (t == 0) {
    int nw = 0;
    for (int u = 0; u < M; ++u) nw += G.key[u];
    G.nwin = nw;
  }
  __syncthreads();
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds + 16*i (lds must be the same for the whole wave).
__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// The base product runs once for all tokens (16-token tiles); the sign
// product once per window: the 16 staged slots starting at the window's first
// slot times the +-1 operand of the window's variant, into the window's own
// accumulator.  Rows of a window past its length hold other tokens' products
// and are never read.  Windows are taken kWin at a time; a batch after the
// first re-streams x and the sign words of its windows but not W_base.
//
// Work split: a workgroup owns 16 output rows; its NW waves take the 128-wide
// blocks of d_in round-robin and their partial sums are added in LDS in a
// fixed order.  Each wave stages its block of x (the MT*16 tokens in variant
// order, 256 bytes each) in its own LDS region with global_load_lds: one
// instruction writes 4 rows, 16 lanes per row (coalesced), and lane (r, c)
// fetches chunk c ^ (r % 16) so that operand reads of 16 consecutive rows at
// one chunk hit distinct banks.  A zero row follows the tokens (windows near
// the end of the batch read it past the last slot).
template <int MT, int NW>
__global__ __launch_bounds__(NW * kWave) void linear_multi_kernel(const SkinnyArgs a) {
  constexpr int kWin = 16;                     // windows per batch
  constexpr int kXRows = MT * 16 + 1;          // token rows + zero row
  constexpr int kXRowB = 256;                  // bytes per staged row (128 bf16)
  constexpr int kXWave = kXRows * kXRowB;
  constexpr int kXBytes = NW * kXWave;
  constexpr int kRedChunk = 8;                 // f32x4 per lane and wave reduced at once
  constexpr int kRedBytes = NW * kRedChunk * 4 * kWave * 4;
  constexpr int kDma = MT * 4;                 // 4-row staging instructions per block
  static_assert(MT <= kRedChunk, "base tiles reduce in one chunk");
  __shared__ __attribute__((aligned(16))) char smem[kRedBytes > kXBytes ? kRedBytes : kXBytes];
  __shared__ Groups G;
  __shared__ float sw_slot[kMaxSkinnyTokens][16];
  __shared__ float ss_slot[kMaxSkinnyTokens][16];

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int d_in = a.d_in;
  const int M = a.M;
  char* xs = smem + wv * kXWave;
  float* red = reinterpret_cast<float*>(smem);

  build_groups(G, a.ids, M, a.n_variants);
  const int nwin = G.nwin;
  const int nbatch = max((nwin + kWin - 1) / kWin, 1);  // one pass at least, for the base
  // Window table, lane w holds window w: first slot and variant.
  const int ws0_l = lane < nwin ? G.ws0[lane] : 0;
  const int wvar_l = lane < nwin ? G.wvar[lane] : 0;

  // Staging sources: instruction j writes rows 4j..4j+3; lane (lane/16,
  // c = lane%16) fetches chunk c ^ (row % 16) of slot row's token (slots past
  // M re-read the last token; their outputs are never stored).  Packed as
  // token | chunk << 8.
  int xsrc[kDma];
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int r = 4 * j + (lane >> 4);
    xsrc[j] = G.perm[min(r, M - 1)] | (((lane & 15) ^ (r & 15)) << 8);
  }
  // Base operand reads: tile t, k-step q, lane (n, g) reads chunk 4g+q of
  // row 16t+n (whose swizzle key is n).
  int foff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) foff[q] = (((4 * g + q) ^ n) << 4);

  const int row0 = blockIdx.x * 16;
  const int row = min(row0 + n, a.d_out - 1);
  const uint16_t* wrow = a.w + (size_t)row * d_in;
  const size_t brow = (size_t)row * (d_in >> 5);

  const int nblk = (d_in + 127) >> 7;
  const int nmine = blocks_of_wave(wv, nblk, NW);
  const bool half_tail = (d_in & 127) != 0;

  f32x4 accw[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) accw[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int batch = 0; batch < nbatch; ++batch) {
    const int wb = batch * kWin;             // first window of the batch
    const int nwb = min(kWin, nwin - wb);    // windows in the batch (<= 0: none)
    f32x4 accv[kWin];
#pragma unroll
    for (int w = 0; w < kWin; ++w) accv[w] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (lane < 16) *reinterpret_cast<u32x4*>(xs + (kXRows - 1) * kXRowB + 16 * lane) = u32x4{0u, 0u, 0u, 0u};

    for (int i = 0; i < nmine; ++i) {
      const int bu = wv + NW * i;
      const int k0 = bu << 7;
      const bool half = half_tail && bu == nblk - 1;  // only its first 64 columns exist
      // x block into LDS (the second half of a half block re-reads the first)
#pragma unroll
      for (int j = 0; j < kDma; ++j) {
        const int ch = xsrc[j] >> 8;
        const int col = k0 + 8 * ch - ((half && ch >= 8) ? 64 : 0);
        lds_load16(a.x + (size_t)(xsrc[j] & 0xFF) * d_in + col, xs + j * 1024);
      }
      const int kc = min(k0 + (g << 5), d_in - 32);
      u32x4 wf[4];
      if (batch == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) wf[q] = ld128(wrow + kc + 8 * q);
      }
      uint32_t sgn[kWin];
#pragma unroll
      for (int w = 0; w < kWin; ++w) {
        if (w < nwb) {
          const int v = __builtin_amdgcn_readlane(wvar_l, wb + w);
          sgn[w] = ld32(a.packed[v] + brow + (kc >> 5));
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      if (half) {
        // columns 64..127 of a half block do not exist: zero them (all rows)
        for (int e = lane; e < (kXRows - 1) * 8; e += kWave) {
          const int r = e >> 3;
          const int cg = 8 + (e & 7);
          *reinterpret_cast<u32x4*>(xs + r * kXRowB + ((cg ^ (r & 15)) << 4)) =
              u32x4{0u, 0u, 0u, 0u};
        }
        __builtin_amdgcn_s_waitcnt(0);
      }
      if (batch == 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const char* src = xs + (16 * t + n) * kXRowB;
          u32x4 xf[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) xf[q] = *reinterpret_cast<const u32x4*>(src + foff[q]);
#pragma unroll
          for (int q = 0; q < 4; ++q) accw[t] = mfma16(xf[q], wf[q], accw[t]);
        }
      }
#pragma unroll
      for (int w = 0; w < kWin; ++w) {
        if (w < nwb) {
          uint32_t sp[16];
          sign_pairs(sgn[w], sp);
          const int r = min(__builtin_amdgcn_readlane(ws0_l, wb + w) + n, MT * 16);
          const char* src = xs + r * kXRowB;
          const int key = r & 15;
          u32x4 xw[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            xw[q] = *reinterpret_cast<const u32x4*>(src + ((((g << 2) + q) ^ key) << 4));
#pragma unroll
          for (int q = 0; q < 4; ++q) accv[w] = mfma16(xw[q], quad(sp, q), accv[w]);
        }
      }
    }

    // Sign sums of the batch's windows: add the waves' partials in a fixed
    // order and file each under its slot.  MFMA 16x16 output layout: lane l
    // holds window rows 4*(l/16)+v of output column l%16.
#pragma unroll
    for (int c0 = 0; c0 < kWin; c0 += kRedChunk) {
      __syncthreads();  // staging (or the previous chunk) no longer read
#pragma unroll
      for (int c = 0; c < kRedChunk; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((wv * kRedChunk + c) * 4 + v) * kWave + lane] = accv[c0 + c][v];
      __syncthreads();
      for (int idx = threadIdx.x; idx < kRedChunk * 4 * kWave; idx += NW * kWave) {
        const int l = idx & (kWave - 1);
        const int v = (idx >> 6) & 3;
        const int c = idx >> 8;
        const int w = wb + c0 + c;
        if (c0 + c < nwb) {
          float ss = 0.f;
#pragma unroll
          for (int k = 0; k < NW; ++k) ss += red[((k * kRedChunk + c) * 4 + v) * kWave + l];
          const int r = 4 * (l >> 4) + v;
          if (r < G.wlen[w]) ss_slot[G.ws0[w] + r][l & 15] = ss;
        }
      }
    }
    if (batch == 0) {
      __syncthreads();
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((wv * kRedChunk + t) * 4 + v) * kWave + lane] = accw[t][v];
      __syncthreads();
      for (int idx = threadIdx.x; idx < MT * 4 * kWave; idx += NW * kWave) {
        const int l = idx & (kWave - 1);
        const int v = (idx >> 6) & 3;
        const int t = idx >> 8;
        float sw = 0.f;
#pragma unroll
        for (int k = 0; k < NW; ++k) sw += red[((k * kRedChunk + t) * 4 + v) * kWave + l];
        const int slot = 16 * t + 4 * (l >> 4) + v;
        if (slot < M) sw_slot[slot][l & 15] = sw;
      }
    }
    __syncthreads();  // the reduction area is the next batch's staging
  }

  const int per_row = a.per_row;
  for (int idx = threadIdx.x; idx < M * 16; idx += NW * kWave) {
    const int slot = idx >> 4;
    const int ol = idx & 15;
    const int o = row0 + ol;
    if (o < a.d_out) {
      const int m = G.perm[slot];
      const int vv = G.slotv[slot];
      const float sw = sw_slot[slot][ol];
      float yv;
      if (vv >= 0) {
        const float* ap = a.alpha[vv];
        yv = sw + (per_row ? ap[o] : ap[0]) * ss_slot[slot][ol];
      } else {
        yv = vv == -1 ? sw : __builtin_nanf("");
      }
      a.y[(size_t)m * a.d_out + o] = f32_to_bf16_bits(yv);
    }
  }
}

// ---------------------------------------------------------------- launchers
constexpr int kNW = 8;

template <int MT, int U>
hipError_t launch_decode(const SkinnyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((linear_decode_kernel<MT, kNW, U>), dim3((a.d_out + 15) / 16),
                     dim3(kNW * kWave), 0, stream, a);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_multi(const SkinnyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((linear_multi_kernel<MT, kNW>), dim3((a.d_out + 15) / 16), dim3(kNW * kWave), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_skinny(const SkinnyArgs& a, hipStream_t stream) {
  // Blocks in flight per wave: 4 for a single token, 2 up to 32 tokens (the
  // x loads grow with the tiles), 1 beyond (measured on 4096x4096).
  if (a.M == 1) return launch_decode<1, 4>(a, stream);
  if (a.M <= 16) return launch_decode<1, 2>(a, stream);
  if (a.M <= 32) return launch_decode<2, 2>(a, stream);
  return launch_decode<4, 1>(a, stream);
}

hipError_t launch_linear_multi(const SkinnyArgs& a, hipStream_t stream) {
  if (a.M <= 16) return launch_multi<1>(a, stream);
  if (a.M <= 32) return launch_multi<2>(a, stream);
  return launch_multi<4>(a, stream);
}

}  // namespace bd
