// Unfused BitDelta on gfx950: the effective weight written to memory.
//
// Page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak", section
// "Sunum mimarisi": the fused kernel forms W_eff = W_base + alpha*sign(Delta)
// in on-chip memory and never writes it out; a server without that kernel
// materialises W_eff in HBM and then runs a standard matmul on it.  This is
// that materialisation, for callers that want a dense W_eff and for timing
// the unfused path against the fused one.  Each element is bf16(W_base +
// alpha_o*s): one float32 addition, then one rounding to bf16 (nearest even),
// computed by the same helper as the prefill GEMM's W_eff tiles, so both hold
// the same bf16 values.
//
// The kernel streams 2 bytes of W_base and 1/8 byte of signs in and 2 bytes
// out per weight.  A workgroup owns one row's block of 256*U pieces of 8
// weights (16 bytes of W_base, one sign byte, 16 bytes of W_eff); thread t
// takes pieces t, t + 256, ..., so every wave instruction reads and writes a
// contiguous 1 KB and the sign bytes 64 contiguous bytes, and all U pieces'
// loads are issued before the first is used.  alpha of the row is one
// scalar load per workgroup.  Pieces past the row re-read the row's last
// piece and are not stored.
#include "common.h"
#include "internal.h"

namespace bd {
namespace {

constexpr int kReconThreads = 256;

template <int U>
__global__ __launch_bounds__(kReconThreads) void reconstruct_kernel(
    const uint16_t* __restrict__ w, const uint8_t* __restrict__ bits8,
    const float* __restrict__ alpha, int per_row, int d_in, int blocks_per_row,
    uint16_t* __restrict__ out) {
  const int row = blockIdx.x / blocks_per_row;
  const int cb = blockIdx.x - row * blocks_per_row;
  const int pieces = d_in >> 3;  // pieces of 8 weights (one sign byte) per row
  const uint32_t ab = __float_as_uint(per_row ? alpha[row] : alpha[0]);
  const size_t r0 = (size_t)row * d_in;
  const uint16_t* wr = w + r0;
  const uint8_t* sr = bits8 + (r0 >> 3);
  uint16_t* orow = out + r0;
  const int p0 = cb * (kReconThreads * U) + threadIdx.x;
  u32x4 wv[U];
  uint32_t sb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = min(p0 + u * kReconThreads, pieces - 1);
    wv[u] = ld128(wr + 8 * p);
    sb[u] = sr[p];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = p0 + u * kReconThreads;
    if (p < pieces) *reinterpret_cast<u32x4*>(orow + 8 * p) = rebuild8(wv[u], sb[u], ab);
  }
}

template <int U>
hipError_t launch_u(const uint16_t* w, const uint8_t* bits8, const float* alpha, int per_row,
                    int d_out, int d_in, uint16_t* out, hipStream_t stream) {
  const int per_block = kReconThreads * U;
  const int blocks_per_row = (d_in / 8 + per_block - 1) / per_block;
  const int64_t grid = (int64_t)d_out * blocks_per_row;
  if (grid > 2147483647) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reconstruct_kernel<U>, dim3((unsigned)grid), dim3(kReconThreads), 0, stream,
                     w, bits8, alpha, per_row, d_in, blocks_per_row, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reconstruct(const uint16_t* w, const uint8_t* packed_bytes, const float* alpha,
                              int per_row, int d_out, int d_in, uint16_t* out,
                              hipStream_t stream) {
  // Pieces in flight per thread: as many as the row holds, up to 4.
  const int pieces = d_in / 8;
  if (pieces >= 4 * kReconThreads)
    return launch_u<4>(w, packed_bytes, alpha, per_row, d_out, d_in, out, stream);
  if (pieces >= 2 * kReconThreads)
    return launch_u<2>(w, packed_bytes, alpha, per_row, d_out, d_in, out, stream);
  return launch_u<1>(w, packed_bytes, alpha, per_row, d_out, d_in, out, stream);
}

}  // namespace bd
