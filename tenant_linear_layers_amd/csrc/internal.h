// Launchers shared between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

constexpr int kMaxVariants = 64;   // equals BITDELTA_MAX_VARIANTS
constexpr int kMaxSkinnyTokens = 64;
// The decode-shaped kernels address a workgroup's 16 rows of W_base and the
// token rows of x (at most 64) with 32-bit buffer offsets: 64 * d_in * 2
// bytes must stay below 2^31.
constexpr int64_t kSkinnyMaxDin = (int64_t(1) << 24) - 64;
// The prefill GEMM addresses one tile's rows of W_base (up to 256 rows) with
// 32-bit buffer offsets: 256 * d_in * 2 bytes must stay below 2^31.
constexpr int64_t kPrefillMaxTileBytes = 2147483647;
constexpr int64_t kPrefillMaxDin = kPrefillMaxTileBytes / (256 * 2) / 64 * 64;

// Compression of one matrix.  per_row != 0: alpha[d_out]; otherwise alpha[1]
// and `partial` holds 2*d_out uint64 of scratch.
hipError_t launch_compress(const uint16_t* w_ft, const uint16_t* w_base, int d_out, int d_in,
                           int per_row, uint64_t* packed, float* alpha, uint64_t* partial,
                           hipStream_t stream);

// Kernel arguments of the decode-shaped linear (single variant or mixed).
struct SkinnyArgs {
  const uint16_t* x;         // [M, d_in]
  const int32_t* ids;        // [M] variant ids (mixed batches only)
  const uint16_t* w;         // [d_out, d_in]
  uint16_t* y;               // [M, d_out]
  int M, d_out, d_in, per_row;
  int n_variants;
  const uint32_t* packed[kMaxVariants];  // packed signs viewed as uint32 words
  const float* alpha[kMaxVariants];
};

// 1 <= M <= 64, one variant (packed[0], alpha[0]).
hipError_t launch_linear_skinny(const SkinnyArgs& a, hipStream_t stream);
// 1 <= M <= 64, token m uses variant ids[m].
hipError_t launch_linear_multi(const SkinnyArgs& a, hipStream_t stream);
// Any M >= 1, one variant; the LDS-staged MFMA GEMM.
hipError_t launch_linear_prefill(const uint16_t* x, int M, const uint16_t* w,
                                 const uint8_t* packed_bytes, const float* alpha, int per_row,
                                 int d_out, int d_in, uint16_t* y, hipStream_t stream);

// W_eff = bf16(W_base + alpha*s) of a whole matrix, written to out
// [d_out, d_in] (the unfused path's materialisation).
hipError_t launch_reconstruct(const uint16_t* w, const uint8_t* packed_bytes, const float* alpha,
                              int per_row, int d_out, int d_in, uint16_t* out,
                              hipStream_t stream);

// MonoSoup merge (rank-r truncations by orthogonal iteration, the mean
// added to the base).  The working width is the rank rounded up to 8, 16 or
// 32; the workspace holds the per-checkpoint bases and partial sums.
int monosoup_width(int rank);
size_t monosoup_workspace_bytes(int64_t d_out, int64_t d_in, int k, int rank);
hipError_t launch_monosoup(const uint16_t* const* w_ft, int k, const uint16_t* w_base, int d_out,
                           int d_in, int rank, int power_iters, const float* omega, uint16_t* out,
                           float* tau, void* workspace, hipStream_t stream);

// Calibration kernels (measured ceilings beside the published peaks).
hipError_t launch_probe_read(const void* src, size_t bytes, int workgroups, uint32_t* sink,
                             hipStream_t stream);
hipError_t launch_probe_mfma(int workgroups, int iters, float* sink, hipStream_t stream);

}  // namespace bd
