// Prefill-shaped BitDelta linear on gfx950: an LDS-staged bf16 MFMA GEMM
// whose weight tiles are rebuilt on the fly from W_base and the sign bits.
//
// Page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak", section
// "Sunum mimarisi": the effective weight W_eff = W_base + alpha*sign(Delta)
// is formed in fast on-chip memory (here LDS) inside the matmul kernel and
// never written to HBM.
//
// Tile: 256 tokens x BN output rows x 64 of d_in per step, WM x WN waves,
// each owning (256/WM) x (BN/WN) outputs in MFMA 32x32x16 tiles (float32
// accumulators in the accumulation registers).  Per step every thread loads
// its share of 16-byte pieces of x and of W_base plus the sign byte of each
// W piece, rebuilds those weights as bf16(W_base + alpha*s) and stores both
// tiles into the second of two LDS buffers while the MFMAs read the first.
// W_eff is rounded to bf16 once per element, the MFMA accumulates in float32
// and y is rounded to bf16.
#include "common.h"
#include "internal.h"

namespace bd {
namespace {

constexpr int BM = 256;
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS row pitch in bf16 (144 bytes) against bank conflicts

// Eight weights of one row: bf16(W_base + alpha*s), s from the sign byte
// (bit j = element j, 1 = +1).  The sign of alpha is flipped by xor for -1.
__device__ __forceinline__ u32x4 rebuild8(u32x4 w, uint32_t byte, uint32_t ab) {
  const uint32_t nb = ~byte;
  u32x4 out;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float lo = __uint_as_float(w[d] << 16);
    const float hi = __uint_as_float(w[d] & 0xFFFF0000u);
    const float slo = __uint_as_float(ab ^ ((nb << (31 - 2 * d)) & 0x80000000u));
    const float shi = __uint_as_float(ab ^ ((nb << (30 - 2 * d)) & 0x80000000u));
    out[d] = pack_bf16x2(lo + slo, hi + shi);
  }
  return out;
}

template <int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void prefill_kernel(
    const uint16_t* __restrict__ x, int M, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ bits8, const float* __restrict__ alpha, int per_row, int d_out,
    int d_in, uint16_t* __restrict__ y, int ntm, int ntn, int chunk) {
  constexpr int NT = 64 * WM * WN;     // threads
  constexpr int RS = NT / 8;           // rows covered by one pass of 16-byte loads
  constexpr int NA = BM / RS;          // x pieces per thread per step
  constexpr int NB = BN / RS;          // W pieces per thread per step
  constexpr int TMW = BM / WM / 32;    // 32-row MFMA tiles per wave
  constexpr int TNW = BN / WN / 32;    // 32-column MFMA tiles per wave
  static_assert(NA >= 1 && NB >= 1 && TMW >= 1 && TNW >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDK];

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous range of tiles, token tile fastest, so tiles that share the
  // same weight tile run under the same L2.
  const int tile = (blockIdx.x & 7) * chunk + (blockIdx.x >> 3);
  if (tile >= ntm * ntn) return;
  const int tm = tile % ntm;
  const int tn = tile / ntm;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int T = threadIdx.x;
  const int lane = T & 63;
  const int wv = T >> 6;
  const int wm = wv % WM;
  const int wn = wv / WM;
  const int lr = T >> 3;   // row within an RS-row slab
  const int lc = T & 7;    // 16-byte chunk within the 64-wide step

  const uint16_t* ap[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) ap[i] = x + (size_t)min(m0 + lr + RS * i, M - 1) * d_in + lc * 8;
  const uint16_t* bp[NB];
  const uint8_t* sp[NB];
  uint32_t ab[NB];
  const size_t bytes_per_row = (size_t)(d_in >> 3);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int r = min(n0 + lr + RS * i, d_out - 1);
    bp[i] = w + (size_t)r * d_in + lc * 8;
    sp[i] = bits8 + (size_t)r * bytes_per_row + lc;
    ab[i] = __float_as_uint(per_row ? alpha[r] : alpha[0]);
  }

  u32x4 ra[NA], rb[NB];
  uint32_t rs[NB];
  auto gload = [&](int kt) {
    const int k = kt * BK;
#pragma unroll
    for (int i = 0; i < NA; ++i) ra[i] = ld128(ap[i] + k);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      rb[i] = ld128(bp[i] + k);
      rs[i] = sp[i][k >> 3];
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < NA; ++i) *reinterpret_cast<u32x4*>(&As[st][lr + RS * i][lc * 8]) = ra[i];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      *reinterpret_cast<u32x4*>(&Bs[st][lr + RS * i][lc * 8]) = rebuild8(rb[i], rs[i], ab[i]);
  };

  f32x16 acc[TMW][TNW];
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = d_in / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kk = ks * 16 + 8 * (lane >> 5);
      u32x4 af[TMW], bf[TNW];
#pragma unroll
      for (int i = 0; i < TMW; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(
            &As[st][wm * (BM / WM) + i * 32 + (lane & 31)][kk]);
#pragma unroll
      for (int j = 0; j < TNW; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(
            &Bs[st][wn * (BN / WN) + j * 32 + (lane & 31)][kk]);
#pragma unroll
      for (int i = 0; i < TMW; ++i)
#pragma unroll
        for (int j = 0; j < TNW; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(st ^ 1);
    __syncthreads();
  }

  // MFMA 32x32 output layout: lane l, element v holds row
  // 8*(v/4) + 4*(l/32) + v%4 of column l%32.
#pragma unroll
  for (int i = 0; i < TMW; ++i) {
#pragma unroll
    for (int j = 0; j < TNW; ++j) {
      const int o = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * (BM / WM) + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M && o < d_out) y[(size_t)m * d_out + o] = f32_to_bf16_bits(acc[i][j][v]);
      }
    }
  }
}

template <int BN, int WM, int WN>
hipError_t launch_cfg(const uint16_t* x, int M, const uint16_t* w, const uint8_t* packed_bytes,
                      const float* alpha, int per_row, int d_out, int d_in, uint16_t* y,
                      hipStream_t stream) {
  const int ntm = (M + BM - 1) / BM;
  const int ntn = (d_out + BN - 1) / BN;
  const int tiles = ntm * ntn;
  const int chunk = (tiles + 7) / 8;
  hipLaunchKernelGGL((prefill_kernel<BN, WM, WN>), dim3(8 * chunk), dim3(64 * WM * WN), 0, stream,
                     x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y, ntm, ntn, chunk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_prefill(const uint16_t* x, int M, const uint16_t* w,
                                 const uint8_t* packed_bytes, const float* alpha, int per_row,
                                 int d_out, int d_in, uint16_t* y, hipStream_t stream) {
  // 8 waves (two per SIMD, so one wave's MFMAs overlap the other's weight
  // rebuild), 256-wide weight tiles when they give at least one tile per CU.
  const long tiles256 = (long)((M + BM - 1) / BM) * ((d_out + 255) / 256);
  if (tiles256 >= 256)
    return launch_cfg<256, 4, 2>(x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y, stream);
  return launch_cfg<128, 4, 2>(x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y, stream);
}

}  // namespace bd
