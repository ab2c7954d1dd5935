// Prefill-shaped BitDelta linear on gfx950: an LDS-staged bf16 MFMA GEMM
// whose weight tiles are rebuilt on the fly from W_base and the sign bits.
//
// Page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak", section
// "Sunum mimarisi": the effective weight W_eff = W_base + alpha*sign(Delta)
// is formed in fast on-chip memory (here LDS) inside the matmul kernel and
// never written to HBM.
//
// Tile: 256 tokens x 128 output rows x 64 of d_in per step, 512 threads
// (8 waves as 4 x 2, each wave 64 x 64 with 2 x 2 MFMA 32x32x16 tiles).
// Each step every thread loads 64 bytes of x and 32 bytes of W_base plus the
// 2 sign bytes that go with them, rebuilds its 16 weights as
// bf16(W_base + alpha*s) and stores both into the second LDS buffer while the
// MFMAs run on the first.  W_eff is rounded to bf16 once per element, the
// MFMA accumulates in float32 and y is rounded to bf16.
#include "common.h"
#include "internal.h"

namespace bd {
namespace {

constexpr int BM = 256;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS row pitch in bf16 (144 bytes) against bank conflicts
constexpr int kThreads = 512;

// Eight weights of one row: bf16(W_base + alpha*s), s from the sign byte
// (bit j = element j, 1 = +1).  The sign of alpha is flipped by xor for -1.
__device__ __forceinline__ u32x4 rebuild8(u32x4 w, uint32_t byte, float alpha) {
  const uint32_t ab = __float_as_uint(alpha);
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

__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const uint16_t* __restrict__ x, int M, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ bits8, const float* __restrict__ alpha, int per_row, int d_out,
    int d_in, uint16_t* __restrict__ y, int ntm, int ntn, int chunk) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDK];

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous range of tiles, token-tile fastest, so tiles that share the
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
  const int wm = wv & 3;
  const int wn = wv >> 2;
  const int lr = T >> 3;  // row within a 64-row slab
  const int lc = T & 7;   // 16-byte chunk within the 64-wide k step

  const uint16_t* ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ap[i] = x + (size_t)min(m0 + lr + 64 * i, M - 1) * d_in + lc * 8;
  const uint16_t* bp[2];
  const uint8_t* sp[2];
  float al[2];
  const size_t bytes_per_row = (size_t)(d_in >> 3);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = min(n0 + lr + 64 * i, d_out - 1);
    bp[i] = w + (size_t)r * d_in + lc * 8;
    sp[i] = bits8 + (size_t)r * bytes_per_row + lc;
    al[i] = per_row ? alpha[r] : alpha[0];
  }

  u32x4 ra[4], rb[2];
  uint32_t rs[2];
  auto gload = [&](int kt) {
    const int k = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ld128(ap[i] + k);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rb[i] = ld128(bp[i] + k);
      rs[i] = sp[i][k >> 3];
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&As[st][lr + 64 * i][lc * 8]) = ra[i];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(&Bs[st][lr + 64 * i][lc * 8]) = rebuild8(rb[i], rs[i], al[i]);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
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
      u32x4 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(&As[st][wm * 64 + i * 32 + (lane & 31)][kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(&Bs[st][wn * 64 + j * 32 + (lane & 31)][kk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(st ^ 1);
    __syncthreads();
  }

  // MFMA 32x32 output layout: lane l, element v holds row
  // 8*(v/4) + 4*(l/32) + v%4 of column l%32.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int o = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M && o < d_out) y[(size_t)m * d_out + o] = f32_to_bf16_bits(acc[i][j][v]);
      }
    }
  }
}

}  // namespace

hipError_t launch_linear_prefill(const uint16_t* x, int M, const uint16_t* w,
                                 const uint8_t* packed_bytes, const float* alpha, int per_row,
                                 int d_out, int d_in, uint16_t* y, hipStream_t stream) {
  const int ntm = (M + BM - 1) / BM;
  const int ntn = (d_out + BN - 1) / BN;
  const int tiles = ntm * ntn;
  const int chunk = (tiles + 7) / 8;
  hipLaunchKernelGGL(prefill_kernel, dim3(8 * chunk), dim3(kThreads), 0, stream, x, M, w,
                     packed_bytes, alpha, per_row, d_out, d_in, y, ntm, ntn, chunk);
  return hipGetLastError();
}

}  // namespace bd
