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
#include <cstdlib>
#include <cstring>

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

// The same operand built one MFMA step at a time: spread_signs gives the two
// spread words, step_signs the four dwords of step q (elements 8q..8q+7).
struct Spread {
  uint32_t zl, zh;
};

__device__ __forceinline__ Spread spread_signs(uint32_t bits) {
  Spread z;
  z.zl = __builtin_amdgcn_bitop3_b32(bits, bits << 15, 0x00005555u, 0x1B);
  z.zh = __builtin_amdgcn_bitop3_b32(bits >> 16, bits >> 1, 0x00005555u, 0x1B);
  return z;
}

__device__ __forceinline__ u32x4 step_signs(const Spread& z, int q) {
  const uint32_t w = q < 2 ? z.zl : z.zh;
  const int i0 = 4 * (q & 1);
  u32x4 v;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    v[k] = __builtin_amdgcn_bitop3_b32(w << (15 - 2 * (i0 + k)), 0x80008000u, 0x3F803F80u, 0xEA);
  return v;
}

__device__ __forceinline__ u32x4 quad(const uint32_t (&s)[16], int q) {
  u32x4 v = {s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
  return v;
}

// Sign words in the operand layout from a coalesced load.  The quad of lanes
// 4r..4r+3 reads row r's 16 bytes (4 sign words) of a block; lane 4r + j
// takes dword sign_quad_dword(4r + j), i.e. dword j for r < 8 and dword
// (j + 2) mod 4 for r >= 8 (the row's two halves swapped).  Lane n + 16g
// then takes dword g of row n from lane sign_perm_src(n, g) by one
// ds_bpermute.  With plain dword j at lane 4r + j, the 32 lanes of each half
// of the wave read source lanes that pair up 32 apart, a two-way bank
// conflict on every permute (measured: one conflict cycle per active LDS
// cycle); with the halves of rows 8..15 swapped they cover all 32 banks.
__device__ __forceinline__ int sign_quad_dword(int lane) {
  return ((lane & 3) + ((lane >> 5) << 1)) & 3;
}
__device__ __forceinline__ int sign_perm_src(int n, int g) {
  return (n << 2) + ((g + ((n >> 3) << 1)) & 3);
}

// Number of a wave's blocks when NW waves take nblk blocks round-robin.
__device__ __forceinline__ int blocks_of_wave(int wv, int nblk, int NW) {
  return wv < nblk ? (nblk - 1 - wv) / NW + 1 : 0;
}

// Sum the NW waves' partial accumulators (LDS, fixed order) and store y.
// rowof(c) is the output row of the workgroup's column c (0..15);
// out(slot, o, sw, ss, m) returns the output value and sets its token m.
template <int MT, int NW, class RowOf, class Out>
__device__ __forceinline__ void reduce_and_store(float* red, const f32x4 (&accw)[MT],
                                                 const f32x4 (&accs)[MT], RowOf rowof, int M,
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
    const int o = rowof(l & 15);
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
  reduce_and_store<MT, NW>(red, accw, accs, [&](int c) { return row0 + c; }, M, a.d_out, a.y,
                           [&](int slot, int o, float sw, float ss, int& m) {
                             m = slot;
                             return sw + (per_row ? alpha[o] : alpha[0]) * ss;
                           });
}

// ---------------------------------------------------------------- one variant, LDS ring
// The same product for M <= 16 with every load coalesced: the address unit
// serves a load whose lanes read contiguous 64-byte pieces four at a time
// (each quad of lanes in one piece) about four times faster than one in the
// MFMA operand layout, where every quad of lanes spans four rows.  So
// W_base and x reach LDS by buffer loads to LDS (4 rows of 256 bytes per
// instruction, chunk c of row r at c ^ (r % 16)) and are read back in the
// operand layout; the sign words are loaded four lanes per row and moved to
// the operand layout by one cross-lane permute.
//
// Each wave owns a ring of U stages (W_base rows of its block, then the x
// rows); the loads of block i + U - 1 are issued before block i is
// multiplied, with a constant count of loads per block, so one vmcnt wait
// finds block i complete.  XD: 4-row x staging instructions per 16-token tile
// (tokens past M re-read the last token; their outputs are never stored).
//
// IL (interleaved rows): workgroup b of G takes four chunks of 4 rows, chunk
// k being rows 4(b + G k) .. 4(b + G k) + 3, instead of rows 16b .. 16b+15,
// and each wave starts at block b mod (its block count) of its range.
// Every row is still taken by exactly one workgroup and one lane column;
// rows past d_out (in the last chunks) read as zero from W_base, re-read the
// last row's signs and are not stored.  W_base is then addressed through one
// resource over the whole matrix, so this needs (d_out + 16) * d_in * 2 <
// 2^31.
// Measured on 4096 x 4096, 8192 x 8192, 10240 x 8192 and 28672 x 8192: 2-7%
// faster at 1 to 16 tokens; on 8192 x 28672 it was 1-3% slower, so it is
// used for d_in up to 8192.
template <int XD, int NW, int U, bool IL>
__global__ __launch_bounds__(NW * kWave) void linear_decode_ring_kernel(const SkinnyArgs a) {
  constexpr int kXR = 4 * XD;                    // staged x rows
  constexpr int kStage = (16 + kXR) * 256;       // W_base rows, then x rows
  constexpr int kLoads = 4 + XD + 1;             // vector loads per block
  constexpr int kRed = NW * 2 * 4 * kWave * 4;   // reduction area (bytes)
  constexpr int kSmem = NW * U * kStage > kRed ? NW * U * kStage : kRed;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int n = lane & 15;
  const int g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int nrows = min(16, a.d_out - row0);
  const int d_in = a.d_in;
  const int M = a.M;
  char* ring = smem + wv * U * kStage;

  // DMA sources, byte offsets at the first block: W_base rows 4j..4j+3 and
  // x rows 4j..4j+3 per instruction, lane (lane/16, c = lane%16) fetching
  // chunk c ^ row.
  // Row of the workgroup's column c (0..15).  G (the grid) from d_out, not
  // gridDim: reading the dispatch packet would delay the first loads.
  const int G = (a.d_out + 15) >> 4;
  auto rowof = [&](int c) { return IL ? 4 * (blockIdx.x + G * (c >> 2)) + (c & 3) : row0 + c; };
  // W_base through one resource: the workgroup's rows, or with IL the whole
  // matrix (below 2^31 bytes; columns past d_out then read as zero).
  const uint16_t* wsrc = IL ? a.w : a.w + (size_t)row0 * d_in;
  const int wbytes = IL ? a.d_out * d_in * 2 : nrows * d_in * 2;
  const int xbytes = M * d_in * 2;
  int wdoff[4], xdoff[XD];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * j + (lane >> 4);
    wdoff[j] = (IL ? rowof(r) : min(r, nrows - 1)) * d_in * 2 + (((lane & 15) ^ r) << 4);
  }
#pragma unroll
  for (int j = 0; j < XD; ++j) {
    const int r = 4 * j + (lane >> 4);
    xdoff[j] = min(r, M - 1) * d_in * 2 + (((lane & 15) ^ r) << 4);
  }
  // Sign words: the quad of lanes 4r..4r+3 loads column r's 16 bytes of the
  // block (halves swapped for r >= 8, see sign_quad_dword).
  const uint8_t* sblk = reinterpret_cast<const uint8_t*>(a.packed[0]) + (IL ? 0 : (size_t)row0 * (d_in >> 3));
  const uint32_t srow = (IL ? min(rowof(lane >> 2), a.d_out - 1) : min(lane >> 2, nrows - 1)) * (d_in >> 3);
  const int sj = sign_quad_dword(lane) << 2;
  const int perm_src = sign_perm_src(n, g) << 2;
  // Operand reads: W row n, x row min(n, kXR - 1), chunk 4g + q.
  const int xr = min(n, kXR - 1);
  int wro[4], xro[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    wro[q] = n * 256 + (((4 * g + q) ^ n) << 4);
    xro[q] = (16 + xr) * 256 + (((4 * g + q) ^ xr) << 4);
  }

  const int nblk = (d_in + 127) >> 7;
  const int nmine = blocks_of_wave(wv, nblk, NW);
  const bool half_tail = (d_in & 127) != 0;

  // Block of the wave's i-th step (IL: rotated by the workgroup index).
  const int rot = IL && nmine > 0 ? (int)(blockIdx.x % (unsigned)nmine) : 0;
  auto blk = [&](int i) { return wv + NW * (i + rot < nmine ? i + rot : i + rot - nmine); };

  uint32_t sreg[U];
  auto issue = [&](int i, int u) {
    const int k0 = blk(i) << 7;
    char* st = ring + u * kStage;
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_bload16(wsrc, wbytes, wdoff[j], 2 * k0, st + j * 1024);
#pragma unroll
    for (int j = 0; j < XD; ++j) lds_bload16(a.x, xbytes, xdoff[j], 2 * k0, st + (16 + 4 * j) * 256);
    const uint32_t off = srow + min((k0 >> 3) + sj, (d_in >> 3) - 4);
    sreg[u] = *reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(
        reinterpret_cast<uintptr_t>(sblk + off));
  };

  f32x4 accw = {0.f, 0.f, 0.f, 0.f}, accs = {0.f, 0.f, 0.f, 0.f};
  if (nmine > 0) {
#pragma unroll
    for (int u = 0; u < U - 1; ++u) issue(min(u, nmine - 1), u);
  }
  for (int i0 = 0; i0 < nmine; i0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u;
      // The stage about to be refilled was read by the previous block: its
      // LDS reads must be complete before the buffer loads may write it (a
      // load to LDS is not ordered after earlier reads of the same wave), and
      // the compiler must not move the loads above this point.
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      // past the wave's last block the issue re-reads that block into a stage
      // nobody reads: every block issues the same number of loads
      issue(min(i + U - 1, nmine - 1), (u + U - 1) % U);
      __builtin_amdgcn_s_waitcnt(((kLoads * (U - 1)) & 15) | (((kLoads * (U - 1)) >> 4) << 14) |
                                 (0x7 << 4) | (0xF << 8));  // vmcnt only
      if (i < nmine) {  // uniform
        char* st = ring + u * kStage;
        if (half_tail && blk(i) == nblk - 1) {
          // a final 64-wide block: zero x's columns 64..127 (read from other bytes)
          for (int e = lane; e < kXR * 8; e += kWave) {
            const int r = e >> 3;
            const int cg = 8 + (e & 7);
            *reinterpret_cast<u32x4*>(st + (16 + r) * 256 + ((cg ^ r) << 4)) =
                u32x4{0u, 0u, 0u, 0u};
          }
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        }
        const uint32_t bits = __builtin_amdgcn_ds_bpermute(perm_src, sreg[u]);
        const Spread z = spread_signs(bits);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 wf = *reinterpret_cast<const u32x4*>(st + wro[q]);
          const u32x4 xf = *reinterpret_cast<const u32x4*>(st + xro[q]);
          accw = mfma16(xf, wf, accw);
          accs = mfma16(xf, step_signs(z, q), accs);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // the ring becomes the reduction area

  float* red = reinterpret_cast<float*>(smem);
  const f32x4 aw[1] = {accw}, as[1] = {accs};
  const float* alpha = a.alpha[0];
  const int per_row = a.per_row;
  reduce_and_store<1, NW>(red, aw, as, rowof, M, a.d_out, a.y,
                          [&](int slot, int o, float sw, float ss, int& m) {
                            m = slot;
                            return sw + (per_row ? alpha[o] : alpha[0]) * ss;
                          });
}

// ---------------------------------------------------------------- one variant, VALU
// The same product for M <= MM <= 4 on the vector ALUs (no matrix cores):
// a workgroup owns 4 output rows and its NW waves take the 128-wide blocks
// of d_in round-robin.  Lane (r = lane/16, c = lane%16) reads 16 bytes of
// W_base row r per block (4 rows of 256 contiguous bytes per load), the
// sign byte of those 8 elements (its quad shares one 4-byte word) and 16
// bytes of each token's x.  Per element: W_base widened to float32 and one
// FMA per token for the base sum; for the sign sum x's sign bit is flipped
// where the sign is -1 (a select by bitop3 on the shifted sign bits) and
// added.  Partial sums are reduced over the 16 lanes of a row by DPP row
// shifts and over the waves in LDS in a fixed order; alpha is applied once.
template <int MM, int NW, int UB>
__global__ __launch_bounds__(NW * kWave) void linear_decode_valu_kernel(const SkinnyArgs a) {
  __shared__ float red[NW][2 * MM][4];

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane >> 4;
  const int c = lane & 15;
  const int d_in = a.d_in;
  const int M = a.M;
  const int row0 = blockIdx.x * 4;
  const int row = min(row0 + r, a.d_out - 1);
  const uint16_t* wrow = a.w + (size_t)row * d_in;
  const uint8_t* srow = reinterpret_cast<const uint8_t*>(a.packed[0]) + (size_t)row * (d_in >> 3);
  const uint16_t* xrow[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) xrow[m] = a.x + (size_t)min(m, M - 1) * d_in;
  const int sbyte = (c & 3) << 3;  // bit offset of the lane's byte in its word

  float aw[MM], as[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) aw[m] = as[m] = 0.f;

  const int nblk = (d_in + 127) >> 7;
  const int nmine = blocks_of_wave(wv, nblk, NW);
  const bool half_tail = (d_in & 127) != 0;
  for (int i0 = 0; i0 < nmine; i0 += UB) {
    u32x4 wv4[UB], xv[UB][MM];
    uint32_t sw[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      // loads are never predicated: past the wave's blocks, and past d_in in
      // a final 64-wide block, they re-read valid bytes that are then skipped
      const int b = wv + NW * min(i0 + u, nmine - 1);
      const int e = min((b << 7) + 8 * c, d_in - 8);  // the lane's first element
      wv4[u] = ld128(wrow + e);
#pragma unroll
      for (int m = 0; m < MM; ++m) xv[u][m] = ld128(xrow[m] + e);
      sw[u] = ld32(srow + ((e >> 3) & ~3));
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (i0 + u >= nmine) continue;  // uniform
      const int b = wv + NW * (i0 + u);
      const bool skip = half_tail && b == nblk - 1 && 8 * c >= 64;
      const uint32_t nb = ~(sw[u] >> sbyte);  // bit j set: element j is -1
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t wd = wv4[u][j >> 1];
        const float w = __uint_as_float((j & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
        const uint32_t neg = nb << (31 - j);
#pragma unroll
        for (int m = 0; m < MM; ++m) {
          const uint32_t xd = xv[u][m][j >> 1];
          const uint32_t xb = (j & 1) ? (xd & 0xFFFF0000u) : (xd << 16);
          const float x = skip ? 0.f : __uint_as_float(xb);
          aw[m] = __builtin_fmaf(w, x, aw[m]);
          // x with its sign bit flipped where the sign is -1 (bitop3 0x78: a ^ (b & c))
          as[m] += __uint_as_float(
              __builtin_amdgcn_bitop3_b32(__float_as_uint(x), neg, 0x80000000u, 0x78));
        }
      }
    }
  }
  // reduce over the 16 lanes of each row (DPP row shifts keep within a row)
#pragma unroll
  for (int m = 0; m < MM; ++m) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
      aw[m] += __shfl_xor(aw[m], off, 16);
      as[m] += __shfl_xor(as[m], off, 16);
    }
  }
  if (c == 0) {
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      red[wv][2 * m][r] = aw[m];
      red[wv][2 * m + 1][r] = as[m];
    }
  }
  __syncthreads();
  if (threadIdx.x < MM * 4) {
    const int m = threadIdx.x >> 2;
    const int rr = threadIdx.x & 3;
    const int o = row0 + rr;
    if (m < M && o < a.d_out) {
      float sw_ = 0.f, ss = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        sw_ += red[w][2 * m][rr];
        ss += red[w][2 * m + 1][rr];
      }
      const float* alpha = a.alpha[0];
      a.y[(size_t)m * a.d_out + o] = f32_to_bf16_bits(sw_ + (a.per_row ? alpha[o] : alpha[0]) * ss);
    }
  }
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
    const int v = ids != nullptr ? ids[t] : 0;  // no ids: every token uses variant 0
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

// ---------------------------------------------------------------- mixed batch, pairs
// Grouping of a mixed batch by (tile, variant) pairs, built once per
// workgroup in LDS.  Tokens are ordered by variant id (stable): slot s holds
// token perm[s] of variant slotv[s] (-1 base only, -2 invalid id), and the
// slots form 16-token tiles (slot s in tile s / 16).  var[0..nvar) are the
// distinct valid variants present, in increasing order.  A pair is one
// variant present in one tile: pair p covers the slots of tile pt[p] that
// hold variant var[pj[p]].  Pairs are listed in slot order, so from one pair
// to the next the tile and the variant index never decrease.
template <int NS>  // slots: M <= NS
struct PairGroups {
  int perm[NS];
  int slotv[NS];
  int key[NS];
  int flag[NS];
  int var[NS];
  int pt[NS];
  int pj[NS];
  int nvar, npair;
};

template <int NS>
__device__ void build_pairs(PairGroups<NS>& G, int vt, int M, int n_variants) {
  const int t = threadIdx.x;
  if (t < M) {
    const int v = vt;  // thread t's token's variant id (0 for a batch without ids)
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
  // key[s] = 1 where slot s starts a variant's run, flag[s] = 1 where it
  // starts a pair (the start of a run, or a tile boundary inside one)
  int v = -3;
  if (t < M) {
    v = G.slotv[t];
    const bool prev_same = t > 0 && G.slotv[t - 1] == v;
    G.key[t] = (v >= 0 && !prev_same) ? 1 : 0;
    G.flag[t] = (v >= 0 && (!prev_same || (t & 15) == 0)) ? 1 : 0;
  }
  __syncthreads();
  if (t < M && v >= 0) {
    int j = -1, p = 0;
    for (int u = 0; u <= t; ++u) j += G.key[u];
    for (int u = 0; u < t; ++u) p += G.flag[u];
    if (G.key[t]) G.var[j] = v;
    if (G.flag[t]) {
      G.pt[p] = t >> 4;
      G.pj[p] = j;
    }
  }
  if (t == 0) {
    int nv = 0, np = 0;
    for (int u = 0; u < M; ++u) {
      nv += G.key[u];
      np += G.flag[u];
    }
    G.nvar = nv;
    G.npair = np;
  }
  __syncthreads();
}

// The base product runs once for all tokens on 16-token tiles; the sign
// product once per pair: x of the pair's tile times the +-1 operand of the
// pair's variant, into the pair's own accumulator.  Rows of a tile that
// belong to other variants get products that are never read.  The tile's x
// operand is read from LDS once per tile change and the +-1 operand is built
// once per variant change (both only move forward along the pair list).
// Pairs are taken KP at a time; a batch after the first re-streams x and the
// sign words of its pairs but not W_base.
//
// Work split: a workgroup owns 16 output rows; its NW waves take the
// 128-wide blocks of d_in round-robin and their partial sums are added in
// LDS in a fixed order.  Lane (n, g) holds elements 32g..32g+31 of the block
// of row n (W_base and sign bits) and of token n of each tile (x).  Per
// block, a wave stages its block of x for the MT*16 slots in its own LDS
// region (buffer loads straight to LDS, 4 rows of 256 bytes per
// instruction; chunk c of row r at c ^ (r % 16), so operand reads of 16
// consecutive rows at one chunk hit distinct banks), and the weights and
// sign words of its next block are requested before the current block is
// multiplied.  The sign rows of the pairs' variants are looked up once per
// batch, outside the loop over blocks.
//
// EW (early weights, for batches with variant ids): the first block of
// W_base does not depend on the grouping, so it is requested into registers
// before the sort (after the token ids, so that waiting for the ids does not
// wait for it) and written to its LDS stage after.  A batch without ids
// sorts at once, and there the wait for these loads before x is requested
// cost 2-3%.
template <int MT, int NW, int KP, bool WLDS, int WPE, bool EARLY, bool EW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(WPE))) void
linear_multi_pairs_kernel(const SkinnyArgs a) {
  static_assert(!EARLY || (MT <= 2 && WLDS), "early staging keeps every tile's x in registers");
  constexpr int kXRows = MT * 16;
  constexpr int kXRowB = 256;                  // bytes per staged row (128 bf16)
  constexpr int kXWave = (kXRows + (WLDS ? 16 : 0)) * kXRowB;  // x rows, then 16 W_base rows
  constexpr int kXBytes = NW * kXWave;
  constexpr int kRedChunk = 8;                 // f32x4 per lane and wave reduced at once
  constexpr int kRedBytes = NW * kRedChunk * 4 * kWave * 4;
  constexpr int kDma = MT * 4;                 // 4-row staging instructions per block
  constexpr int kSmem = kRedBytes > kXBytes ? kRedBytes : kXBytes;
  static_assert(MT <= kRedChunk, "base tiles reduce in one chunk");
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  __shared__ PairGroups<kXRows> G;
  __shared__ float sw_slot[kXRows][16];
  __shared__ float ss_slot[kXRows][16];

  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int n = lane & 15;
  const int g = lane >> 4;
  const int d_in = a.d_in;
  const int M = a.M;
  char* xs = smem + wv * kXWave;
  char* ws = xs + kXRows * kXRowB;  // the wave's 16 rows of W_base for one block
  float* red = reinterpret_cast<float*>(smem);

  // Token ids first (no branch around the load, so that the compiler counts
  // the loads issued after it exactly).
  const int vt = a.ids != nullptr ? a.ids[min((int)threadIdx.x, M - 1)] : 0;
  const int row0 = blockIdx.x * 16;
  const int nrows = min(16, a.d_out - row0);
  const uint16_t* wblk = a.w + (size_t)row0 * d_in;
  const int wbytes = nrows * d_in * 2;
  // W_base staging (WLDS), like x: instruction j writes rows 4j..4j+3 of
  // the block, lane (lane/16, c = lane%16) fetching chunk c ^ row of its row
  // (rows past d_out re-read the last row).  Byte offsets at the first
  // block.  Without WLDS the lane loads its own 64 bytes in operand layout.
  const int woff = (min(n, nrows - 1) * d_in + (g << 5)) * 2;  // + 2*k0 per block
  int wdoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * j + (lane >> 4);
    wdoff[j] = min(r, nrows - 1) * d_in * 2 + (((lane & 15) ^ r) << 4);
  }
  const int nblk = (d_in + 127) >> 7;
  const int nmine = blocks_of_wave(wv, nblk, NW);
  u32x4 w0[4];
  if (EW) {
    // the first block of W_base (a wave with no blocks reads zeros past d_in)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w0[j] = WLDS ? bload128(wblk, wbytes, wdoff[j], 2 * (wv << 7))
                   : bload128(wblk, wbytes, woff + 16 * j, 2 * (wv << 7));
  }
  build_pairs(G, vt, M, a.n_variants);
  if (EW && WLDS) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(ws + j * 1024 + (lane << 4)) = w0[j];
  }
  const int npair = G.npair;
  const int nbatch = max((npair + KP - 1) / KP, 1);  // one pass at least, for the base
  // Pair and variant tables, lane p holding entry p.
  const int pt_l = lane < npair ? G.pt[lane] : 0;
  const int pj_l = lane < npair ? G.pj[lane] : -1;

  // Staging: instruction j writes slot rows 4j..4j+3; lane (lane/16,
  // c = lane%16) fetches chunk c ^ (row % 16) of the row's token (slots past
  // M re-read the last token; their outputs are never stored).  Byte offsets
  // into x at the first block.
  const int xbytes = M * d_in * 2;
  int xoff[kDma];
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int r = 4 * j + (lane >> 4);
    xoff[j] = G.perm[min(r, M - 1)] * d_in * 2 + (((lane & 15) ^ (r & 15)) << 4);
  }
  // Operand reads: tile t, k-step q, lane (n, g) reads chunk 4g+q of slot
  // row 16t+n (whose swizzle key is n).
  int foff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) foff[q] = (((4 * g + q) ^ n) << 4);

  // Sign words are loaded with four lanes per row (the quad of lanes
  // 4r..4r+3 reads row r's 16 bytes of the block: every quad of lanes reads
  // one contiguous piece, which the address unit serves four times faster
  // than the operand layout), then moved to the operand layout (lane n + 16g
  // holds dword g of row n) by one cross-lane permute (sign_quad_dword).
  const uint32_t srow = min(lane >> 2, nrows - 1) * (d_in >> 3);
  const int sj = sign_quad_dword(lane) << 2;
  const int perm_src = sign_perm_src(n, g) << 2;       // byte address of the source lane
  const size_t prow = (size_t)row0 * (d_in >> 3);      // this workgroup's rows in a packed matrix

  const bool half_tail = (d_in & 127) != 0;

  f32x4 accw[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) accw[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int batch = 0; batch < nbatch; ++batch) {
    const int p0 = batch * KP;
    const int np = min(KP, npair - p0);  // pairs in the batch (<= 0: none)
    // Lane u: the sign rows (this workgroup's) of pair p0+u's variant.
    const uint8_t* stab = nullptr;
    if (lane < np) {
      const int vv = G.var[G.pj[p0 + lane]];
      stab = reinterpret_cast<const uint8_t*>(a.packed[vv]) + prow;
    }
    const uint64_t stab_u = reinterpret_cast<uint64_t>(stab);
    const uint32_t stab_lo = (uint32_t)stab_u, stab_hi = (uint32_t)(stab_u >> 32);
    // Pair u builds a +-1 operand (and so needs its sign words) when it
    // starts a new variant; otherwise it reuses the previous pair's.
    const int jprev_l = __shfl_up(pj_l, 1, kWave);
    const uint64_t builds = __builtin_amdgcn_ballot_w64(
        lane >= p0 && lane < p0 + np && (lane == p0 || pj_l != jprev_l));

    f32x4 acc[KP];
#pragma unroll
    for (int u = 0; u < KP; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint32_t sc[KP];
    u32x4 wc[4];
    if (EW && !WLDS && batch == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) wc[q] = w0[q];
    }
    auto stage_w = [&](int i) {
      const int k0 = (wv + NW * i) << 7;
      if (WLDS) {
#pragma unroll
        for (int j = 0; j < 4; ++j) lds_bload16(wblk, wbytes, wdoff[j], 2 * k0, ws + j * 1024);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) wc[q] = bload128(wblk, wbytes, woff + 16 * q, 2 * k0);
      }
    };
    auto sign_word = [&](int i, int u) -> uint32_t {
      // dword sj/4 of the row's 16 sign bytes of block wv + NW*i; in a final
      // 64-wide block dwords 2 and 3 re-read the row's last 4 bytes (never
      // past the row)
      const uint32_t off = srow + min(((wv + NW * i) << 4) + sj, (d_in >> 3) - 4);
      const uint64_t b = ((uint64_t)__builtin_amdgcn_readlane(stab_hi, u) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane(stab_lo, u);
      return *reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(b + off);
    };
    auto load_s1 = [&](int i, int u) { sc[u] = sign_word(i, u); };
    auto stage_x = [&](int i) {
      const int k0 = (wv + NW * i) << 7;
#pragma unroll
      for (int j = 0; j < kDma; ++j) lds_bload16(a.x, xbytes, xoff[j], 2 * k0, xs + j * 1024);
    };
    if constexpr (EARLY) {
      // Every load of block i+1 is issued at the top of block i: its x once
      // all tiles' x operands of block i are in registers, its sign words
      // into sn, its W_base once this block's W operand is in registers.
      // The sign words are moved into the operand layout at the end of the
      // block.
      uint32_t sn[KP];
#pragma unroll
      for (int u = 0; u < KP; ++u) sn[u] = 0u;
      if (nmine > 0) {
        stage_x(0);
        if (batch == 0 && !EW) stage_w(0);
#pragma unroll
        for (int u = 0; u < KP; ++u)
          if ((builds >> (p0 + u)) & 1) sn[u] = sign_word(0, u);
#pragma unroll
        for (int u = 0; u < KP; ++u) sc[u] = __builtin_amdgcn_ds_bpermute(perm_src, sn[u]);
      }
      for (int i = 0; i < nmine; ++i) {
        __builtin_amdgcn_s_waitcnt(0);  // x and W_base of block i staged
        const bool more = i + 1 < nmine;
        const int inext = more ? i + 1 : i;
        if (half_tail && wv + NW * i == nblk - 1) {
          // a final 64-wide block: zero columns 64..127 of every slot row
          for (int e = lane; e < kXRows * 8; e += kWave) {
            const int r = e >> 3;
            const int cg = 8 + (e & 7);
            *reinterpret_cast<u32x4*>(xs + r * kXRowB + ((cg ^ (r & 15)) << 4)) =
                u32x4{0u, 0u, 0u, 0u};
          }
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        }
        u32x4 xt[MT][4];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const char* src = xs + (16 * t + n) * kXRowB;
#pragma unroll
          for (int q = 0; q < 4; ++q) xt[t][q] = *reinterpret_cast<const u32x4*>(src + foff[q]);
        }
        u32x4 wf[4];
        if (batch == 0) {
          const char* src = ws + n * kXRowB;
#pragma unroll
          for (int q = 0; q < 4; ++q) wf[q] = *reinterpret_cast<const u32x4*>(src + foff[q]);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): both stages read
        if (more) stage_x(i + 1);
#pragma unroll
        for (int u = 0; u < KP; ++u)
          if ((builds >> (p0 + u)) & 1) sn[u] = sign_word(inext, u);
        if (batch == 0) {
#pragma unroll
          for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) accw[t] = mfma16(xt[t][q], wf[q], accw[t]);
          if (more) stage_w(inext);
        }
        Spread sz;
#pragma unroll
        for (int u = 0; u < KP; ++u) {
          if (u < np) {
            const int t = __builtin_amdgcn_readlane(pt_l, p0 + u);
            if ((builds >> (p0 + u)) & 1) sz = spread_signs(sc[u]);
            if (MT == 1 || t == 0) {
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[u] = mfma16(xt[0][q], step_signs(sz, q), acc[u]);
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                acc[u] = mfma16(xt[MT - 1][q], step_signs(sz, q), acc[u]);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < KP; ++u) sc[u] = __builtin_amdgcn_ds_bpermute(perm_src, sn[u]);
      }
    } else {
    if (nmine > 0) {
      stage_x(0);
      if (batch == 0 && !EW) stage_w(0);
#pragma unroll
      for (int u = 0; u < KP; ++u)
        if ((builds >> (p0 + u)) & 1) load_s1(0, u);
    }
    for (int i = 0; i < nmine; ++i) {
      __builtin_amdgcn_s_waitcnt(0);  // x staged, weights and sign words of block i
      const bool more = i + 1 < nmine;
      if (half_tail && wv + NW * i == nblk - 1) {
        // a final 64-wide block: its columns 64..127 do not exist (the
        // staging read other bytes there): zero them in every slot row, so
        // that they add nothing whatever the weights and signs read there
        for (int e = lane; e < kXRows * 8; e += kWave) {
          const int r = e >> 3;
          const int cg = 8 + (e & 7);
          *reinterpret_cast<u32x4*>(xs + r * kXRowB + ((cg ^ (r & 15)) << 4)) =
              u32x4{0u, 0u, 0u, 0u};
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      }
      u32x4 xw[4];
      auto read_x = [&](int t) {
        const char* src = xs + (16 * t + n) * kXRowB;
#pragma unroll
        for (int q = 0; q < 4; ++q) xw[q] = *reinterpret_cast<const u32x4*>(src + foff[q]);
      };
      // The next block's W_base goes into the W stage once this block's has
      // been read, and each sign word into its register right after its last
      // use (the last block re-reads itself: no register load depends on a
      // condition, which would make the compiler wait for it before the
      // merge).
      const int inext = more ? i + 1 : i;
      // this block's sign words into the operand layout
      // (every slot: a slot that loaded nothing permutes a stale word it never reads)
#pragma unroll
      for (int u = 0; u < KP; ++u) sc[u] = __builtin_amdgcn_ds_bpermute(perm_src, sc[u]);
      int tcur = -1;
      if (batch == 0) {
        u32x4 wf[4];
        if (WLDS) {
          const char* src = ws + n * kXRowB;
#pragma unroll
          for (int q = 0; q < 4; ++q) wf[q] = *reinterpret_cast<const u32x4*>(src + foff[q]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) wf[q] = wc[q];
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          read_x(t);
#pragma unroll
          for (int q = 0; q < 4; ++q) accw[t] = mfma16(xw[q], wf[q], accw[t]);
        }
        tcur = MT - 1;
        if (WLDS) {
          if (more) {
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the W stage has been read
            stage_w(inext);
          }
        } else {
          stage_w(inext);  // wc is free again
        }
      }
      Spread sz;
#pragma unroll
      for (int u = 0; u < KP; ++u) {
        if (u < np) {
          const int t = __builtin_amdgcn_readlane(pt_l, p0 + u);
          if (t != tcur) {
            tcur = t;
            read_x(t);
          }
          if ((builds >> (p0 + u)) & 1) {
            sz = spread_signs(sc[u]);
            // keep the reload of sc[u] after its last read, so that it lands
            // in the same register with no copy (and no wait for the copy)
            __builtin_amdgcn_sched_barrier(0);
            load_s1(inext, u);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[u] = mfma16(xw[q], step_signs(sz, q), acc[u]);
        }
      }
      if (more) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this block's LDS reads are done
        stage_x(i + 1);
      }
    }
    }

    // Sign sums of the batch's pairs: add the waves' partials in a fixed
    // order and file each under the slots of its tile that hold its
    // variant.  MFMA 16x16 output layout: lane l holds tile rows
    // 4*(l/16)+v of output column l%16.
#pragma unroll
    for (int c0 = 0; c0 < KP; c0 += kRedChunk) {
      __syncthreads();  // staging (or the previous chunk) no longer read
#pragma unroll
      for (int c = 0; c < kRedChunk; ++c)
        if (c0 + c < KP)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            red[((wv * kRedChunk + c) * 4 + v) * kWave + lane] = acc[min(c0 + c, KP - 1)][v];
      __syncthreads();
      for (int idx = threadIdx.x; idx < kRedChunk * 4 * kWave; idx += NW * kWave) {
        const int l = idx & (kWave - 1);
        const int v = (idx >> 6) & 3;
        const int c = idx >> 8;
        const int u = c0 + c;
        if (u < KP && u < np) {
          float ss = 0.f;
#pragma unroll
          for (int k = 0; k < NW; ++k) ss += red[((k * kRedChunk + c) * 4 + v) * kWave + l];
          const int slot = 16 * G.pt[p0 + u] + 4 * (l >> 4) + v;
          if (slot < M && G.slotv[slot] == G.var[G.pj[p0 + u]]) ss_slot[slot][l & 15] = ss;
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

// Environment switches for A/B measurements of alternative kernels, read at
// every call (a lookup is far cheaper than a launch).
bool env_is(const char* name, const char* value) {
  const char* e = std::getenv(name);
  return e != nullptr && std::strcmp(e, value) == 0;
}

template <int MM, int NW, int UB>
hipError_t launch_decode_valu(const SkinnyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((linear_decode_valu_kernel<MM, NW, UB>), dim3((a.d_out + 3) / 4),
                     dim3(NW * kWave), 0, stream, a);
  return hipGetLastError();
}

// The vector-ALU GEMV for M <= 4 (BITDELTA_DECODE_KERNEL=valu).
bool decode_use_valu() { return env_is("BITDELTA_DECODE_KERNEL", "valu"); }

template <int XD, int NW, int U>
hipError_t launch_decode_ring(const SkinnyArgs& a, hipStream_t stream) {
  // interleaved rows reach d_out + 14: their offsets stay below 2^31
  if (a.d_in <= 8192 && ((int64_t)a.d_out + 16) * a.d_in * 2 < (int64_t(1) << 31))
    hipLaunchKernelGGL((linear_decode_ring_kernel<XD, NW, U, true>), dim3((a.d_out + 15) / 16),
                       dim3(NW * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((linear_decode_ring_kernel<XD, NW, U, false>), dim3((a.d_out + 15) / 16),
                       dim3(NW * kWave), 0, stream, a);
  return hipGetLastError();
}

// The earlier decode kernel (operand-layout loads) for every M
// (BITDELTA_DECODE_KERNEL=operand).
bool decode_use_old() { return env_is("BITDELTA_DECODE_KERNEL", "operand"); }

template <int MT>
hipError_t launch_multi(const SkinnyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((linear_multi_kernel<MT, kNW>), dim3((a.d_out + 15) / 16), dim3(kNW * kWave), 0,
                     stream, a);
  return hipGetLastError();
}

template <int MT, int NW, int KP, bool WLDS, int WPE, bool EARLY>
hipError_t launch_multi_pairs(const SkinnyArgs& a, hipStream_t stream) {
  if (a.ids != nullptr)
    hipLaunchKernelGGL((linear_multi_pairs_kernel<MT, NW, KP, WLDS, WPE, EARLY, true>),
                       dim3((a.d_out + 15) / 16), dim3(NW * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((linear_multi_pairs_kernel<MT, NW, KP, WLDS, WPE, EARLY, false>),
                       dim3((a.d_out + 15) / 16), dim3(NW * kWave), 0, stream, a);
  return hipGetLastError();
}

// Which mixed-batch kernel runs: pairs (default) or windows
// (BITDELTA_MULTI_KERNEL=windows).
bool multi_use_windows() { return env_is("BITDELTA_MULTI_KERNEL", "windows"); }

}  // namespace

// The (tile, variant) pairs kernel for a batch of M tokens.
hipError_t launch_multi_tiles(const SkinnyArgs& a, hipStream_t stream) {
  // Four waves per workgroup (three workgroups per CU) where there are at
  // least 320 groups of 16 rows; eight otherwise (measured: 28672 x 8192 at
  // 32 tokens 246 against 265 us, 8192 x 8192 76 us, 5120 x 4096 at 16 and
  // 32 tokens 26.9 and 38.6 against 31.0 and 44.6 us; with 256 groups, 4096
  // x 4096 at 16 tokens, 25.0 against 21.8 us).
  // Early staging (every load of the next block issued at the top of the
  // current one) for one token tile: 28672 x 8192 at 16 tokens 165 -> 157
  // us.  At two tiles it needs 32 more registers a lane: with three
  // workgroups per CU they spill (472 us), with two it is no faster (246
  // against 242 us).
  const bool wide = (a.d_out + 15) / 16 >= 320;
  if (a.M <= 16)
    return wide ? launch_multi_pairs<1, 4, 12, true, 3, true>(a, stream)
                : launch_multi_pairs<1, 8, 12, true, 2, true>(a, stream);
  if (a.M <= 32)
    return wide ? launch_multi_pairs<2, 4, 12, true, 3, false>(a, stream)
                : launch_multi_pairs<2, 8, 12, true, 2, false>(a, stream);
  // Up to 64 tokens: two workgroups of four waves per CU (75.5 KB of LDS
  // each, 16 pairs per batch) where there are at least 320 row groups, else
  // one of eight waves.  Four waves: 28672 x 8192 at 64 tokens 380 -> 340
  // us, at 48 tokens 356 -> 316 us, 8192 x 8192 113 -> 105 us, 5120 and
  // 6144 x 4096 68 -> 58 us, 8192 x 28672 363 -> 357 us; with 256 row
  // groups (4096 x 4096) it was 22% slower (one workgroup, four waves a CU).
  if ((a.d_out + 15) / 16 >= 320) return launch_multi_pairs<4, 4, 16, false, 2, false>(a, stream);
  return launch_multi_pairs<4, 8, 20, false, 2, false>(a, stream);
}

hipError_t launch_linear_skinny(const SkinnyArgs& a, hipStream_t stream) {
  if (decode_use_valu() && a.M <= 4) {
    if (a.M == 1) return launch_decode_valu<1, 4, 16>(a, stream);
    if (a.M == 2) return launch_decode_valu<2, 4, 4>(a, stream);
    return launch_decode_valu<4, 4, 4>(a, stream);
  }
  // Two ring stages; up to 8 tokens eight waves (80 and 96 KB of LDS per
  // workgroup, measured on 4096 x 4096, 28672 x 8192 and 8192 x 28672),
  // but four (half the LDS, twice the blocks per wave) where the row groups
  // number 256..320: 4096 x 4096 at 1 / 4 / 8 tokens 8.72 / 8.87 / 9.25 ->
  // 8.49 / 8.57 / 8.70 us, 5120 x 4096 12.6 -> 12.1 us, 4096 x 8192 14.55
  // -> 14.2 us.  With 128 or fewer groups (2048 rows: 6.7 -> 7.1 us) and
  // with 512 or 640 (8192, 10240 rows: 2-4% slower) eight waves stay
  // faster; at 384 (6144 rows) it went either way (-1.8% with d_in 4096,
  // +1.3% with 8192).
  if (!decode_use_old() && a.M <= 16) {
    const int groups = (a.d_out + 15) / 16;
    const bool four = groups >= 256 && groups <= 320;
    if (a.M <= 4)
      return four ? launch_decode_ring<1, 4, 2>(a, stream) : launch_decode_ring<1, 8, 2>(a, stream);
    if (a.M <= 8)
      return four ? launch_decode_ring<2, 4, 2>(a, stream) : launch_decode_ring<2, 8, 2>(a, stream);
    // 9..16 tokens: four waves with two stages (64 KB, two workgroups per
    // CU) rather than eight with one: 4096 x 4096 9.38-9.45 -> 9.29 us,
    // 28672 x 8192 98.1 -> 96.6 us, 8192 x 8192 and 10240 x 8192 equal.
    return launch_decode_ring<4, 4, 2>(a, stream);
  }
  // Beyond 16 tokens the pairs kernel with every token on variant 0 (no
  // ids): 10-35% faster than the operand-layout decode kernel from 24 to 64
  // tokens on 28672 x 8192, 8192 x 8192 and 8192 x 28672 (28672 x 8192 at
  // 32 tokens 185 -> 154 us).
  if (!decode_use_old()) {
    SkinnyArgs b = a;
    b.ids = nullptr;
    b.n_variants = 1;
    return launch_multi_tiles(b, stream);
  }
  // Blocks in flight per wave: 4 for a single token, 2 up to 32 tokens (the
  // x loads grow with the tiles), 1 beyond (measured on 4096x4096).
  if (a.M == 1) return launch_decode<1, 4>(a, stream);
  if (a.M <= 16) return launch_decode<1, 2>(a, stream);
  if (a.M <= 32) return launch_decode<2, 2>(a, stream);
  return launch_decode<4, 1>(a, stream);
}

hipError_t launch_linear_multi(const SkinnyArgs& a, hipStream_t stream) {
  if (multi_use_windows()) {
    if (a.M <= 16) return launch_multi<1>(a, stream);
    if (a.M <= 32) return launch_multi<2>(a, stream);
    return launch_multi<4>(a, stream);
  }
  return launch_multi_tiles(a, stream);
}

}  // namespace bd
