// BitDelta compression on gfx950: Delta = W_ft - W_base, packed sign(Delta)
// and alpha = mean|Delta|, in one HBM-streaming pass.
//
// Page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak": section
// "Matematiksel temel" (Delta, the sign code and the alpha equation) and
// section "Altyapı ayrıntıları" (signs stored 8 per byte along the input
// dimension, alpha as float32).
//
// One wave per row.  Lane k of a wave reads 16 bytes of each input per
// 512-element chunk (elements 8k..8k+7), so every wave-wide load is a
// contiguous 1 KiB.  The lane's eight signs are exactly byte k of the chunk's
// packed bits (least significant bit first), which the lane stores itself.
// The scale is summed exactly in integers (floor(|d| * 2^48)), so the result
// does not depend on the order of summation.
#include "common.h"
#include "internal.h"
#include "scale_round.h"

#pragma clang fp contract(off)

namespace bd {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row, 256 threads

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Exact per-lane sum of floor(|d| * 2^48) over the lane's elements of one
// row, by the two-limb method (hi = floor(|d| * 2^16), lo = the next 32
// fraction bits), safe for any |d| < 2^15; *bad is set for larger, infinite
// or NaN deltas.  Used for rows whose largest |d| is too big for the fast
// single-sum path below.
struct RowSum {
  uint64_t hi, lo;
  uint32_t bad;
};

__device__ __forceinline__ RowSum row_sum_two_limbs(const uint16_t* a_row, const uint16_t* b_row,
                                                    int d_in, int lane) {
  uint64_t acc_hi = 0, acc_lo = 0;
  uint32_t b = 0;
  for (int e0 = lane << 3; e0 < d_in; e0 += 512) {
    const u32x4 va = ld128(a_row + e0);
    const u32x4 vb = ld128(b_row + e0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t ua = (j & 1) ? (va[j >> 1] & 0xFFFF0000u) : (va[j >> 1] << 16);
      const uint32_t ub = (j & 1) ? (vb[j >> 1] & 0xFFFF0000u) : (vb[j >> 1] << 16);
      const float d = __uint_as_float(ua) - __uint_as_float(ub);
      float ad = __builtin_fabsf(d) * 65536.0f;
      const bool ok = ad < 2147483648.0f;  // false for NaN, inf, |d| >= 2^15
      b |= ok ? 0u : 1u;
      ad = ok ? ad : 0.0f;
      const uint32_t hi = (uint32_t)ad;
      const uint32_t lo = (uint32_t)((ad - (float)hi) * 4294967296.0f);
      acc_hi += hi;
      acc_lo += lo;
    }
  }
  RowSum r;
  r.hi = wave_sum_u64(acc_hi);
  r.lo = wave_sum_u64(acc_lo);
  r.bad = __builtin_amdgcn_ballot_w64(b != 0) != 0;
  return r;
}

// Per-row pass.  kPerRow: write alpha[row] directly; otherwise write the
// row's sum as two limbs to partial[2*row .. 2*row+1] (S = hi * 2^32 + lo; a
// row with a bad delta gets hi = ~0).
//
// Fast path: q = floor(|d| * 2^48) is the 64-bit pair (lo, hi) of the two
// exact conversions hi = floor(|d| * 2^16) and lo = floor(frac(|d| * 2^16) *
// 2^32), and the row's sum of q fits 64 bits whenever max|d| * 2^48 * d_in <
// 2^64: each element costs one 64-bit add and one max of |d|'s bits (the
// range check is done once per row from that maximum).  A row failing the
// bound is summed again by the two-limb method.
template <bool kPerRow>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void compress_rows_kernel(
    const uint16_t* __restrict__ w_ft, const uint16_t* __restrict__ w_base, int d_out, int d_in,
    uint64_t* __restrict__ packed, float* __restrict__ alpha, uint64_t* __restrict__ partial) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= d_out) return;  // whole wave leaves together

  const uint16_t* a_row = w_ft + (size_t)row * d_in;
  const uint16_t* b_row = w_base + (size_t)row * d_in;
  uint8_t* p_bytes = reinterpret_cast<uint8_t*>(packed) + (size_t)row * (d_in >> 3);

  // Row sum of q = hi * 2^32 + lo as a (acc_lo, acc_hi) pair: one add with
  // carry-out and one add with carry-in per element.
  uint32_t acc_lo = 0, acc_hi = 0;
  uint32_t maxbits = 0;  // largest float bits of |d| * 2^16 (NaN bits sort above inf)
  const int n_chunks = (d_in + 511) >> 9;
  const int n_full = d_in >> 9;  // chunks with all 512 elements present

  // Sign byte, magnitude sum and running maximum of one chunk's 8 elements
  // per lane.
  auto chunk = [&](const u32x4& va, const u32x4& vb) -> uint32_t {
    uint32_t sbyte = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t ua = (j & 1) ? (va[j >> 1] & 0xFFFF0000u) : (va[j >> 1] << 16);
      const uint32_t ub = (j & 1) ? (vb[j >> 1] & 0xFFFF0000u) : (vb[j >> 1] << 16);
      const float d = __uint_as_float(ua) - __uint_as_float(ub);
      // sign bit 1 <=> +1 <=> not (d < 0): +0, -0 and NaN give +1.
      sbyte |= (d < 0.0f) ? 0u : (1u << j);
      const float ad = __builtin_fabsf(d) * 65536.0f;
      maxbits = max(maxbits, __float_as_uint(ad));
      // Conversions saturate for out-of-range values; such rows are
      // recomputed or flagged below, so their sum here is discarded.
      const uint32_t hi = (uint32_t)ad;
      const uint32_t lo = (uint32_t)(__builtin_amdgcn_fractf(ad) * 4294967296.0f);
      const uint32_t nl = acc_lo + lo;
      acc_hi += hi + (nl < lo ? 1u : 0u);
      acc_lo = nl;
    }
    return sbyte;
  };

  // Four chunks per group: all eight 16-byte loads of a group are issued
  // before any is used (8 KiB per wave in flight; 16 KiB measured slower),
  // and each chunk is processed as soon as its own loads have arrived.
  constexpr int kGroup = 4;
  for (int c0 = 0; c0 < n_chunks; c0 += kGroup) {
    // Loads are never predicated (see the decode kernel): lanes past the end
    // of the row re-read its last 16 bytes and are zeroed afterwards, which
    // only happens in a final partial chunk (d_in % 512 != 0).
    u32x4 va[kGroup], vb[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int e0 = min(((c0 + u) << 9) + (lane << 3), d_in - 8);
      va[u] = ld128(a_row + e0);
      vb[u] = ld128(b_row + e0);
    }
    // Byte `lane` of a chunk's 64 packed bytes holds its elements
    // 8*lane .. 8*lane+7 (bit j = element 8*lane+j): one byte store per
    // lane, 64 contiguous bytes per wave.
    if (c0 + kGroup <= n_full) {  // uniform: a group of whole chunks, no checks
#pragma unroll
      for (int u = 0; u < kGroup; ++u)
        p_bytes[((c0 + u) << 6) + lane] = (uint8_t)chunk(va[u], vb[u]);
    } else {
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        const int c = c0 + u;
        if (c >= n_chunks) continue;  // uniform
        if (c >= n_full && (c << 9) + (lane << 3) >= d_in) {
          // d_in is a multiple of 64, so the active lanes of a partial chunk
          // cover whole 64-element words; the rest contribute +1 signs
          // (never stored) and zero magnitudes.
          va[u] = u32x4{0u, 0u, 0u, 0u};
          vb[u] = u32x4{0u, 0u, 0u, 0u};
        }
        const uint32_t sbyte = chunk(va[u], vb[u]);
        if ((c << 9) + (lane << 3) < d_in) p_bytes[(c << 6) + lane] = (uint8_t)sbyte;
      }
    }
  }
  const uint64_t acc = ((uint64_t)acc_hi << 32) | acc_lo;

  // Row-wide largest |d| * 2^16 (float bits; the values are >= 0, so their
  // bit patterns order like the values, and NaN patterns sort above inf).
  uint32_t mb = maxbits;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, off, 64));
  // Fast path valid iff max|d| * 2^16 * d_in < 2^32, i.e. the row sum of q
  // stays below 2^64; checked in float without rounding trouble since d_in
  // is a power-of-two multiple of 64 times an integer < 2^31.
  const float maxad = __uint_as_float(mb);
  const bool row_bad_fast = !(maxad < 2147483648.0f);  // also NaN, inf
  const bool fast = !row_bad_fast && maxad * (float)d_in < 4294967296.0f * 0.5f;
  uint64_t s_hi, s_lo;
  uint32_t row_bad;
  if (fast) {
    const uint64_t s = wave_sum_u64(acc);
    s_hi = s >> 32;
    s_lo = s & 0xFFFFFFFFull;
    row_bad = 0;
  } else if (row_bad_fast) {
    s_hi = s_lo = 0;
    row_bad = 1;
  } else {
    const RowSum r = row_sum_two_limbs(a_row, b_row, d_in, lane);
    s_hi = r.hi;
    s_lo = r.lo;
    row_bad = r.bad;
  }
  if (lane == 0) {
    if (kPerRow) {
      // S = s_hi * 2^32 + s_lo as a 128-bit value.
      const uint64_t lo = (s_hi << 32) + s_lo;
      const uint64_t hi = (s_hi >> 32) + (lo < s_lo ? 1u : 0u);
      const uint32_t bits = row_bad ? 0x7FC00000u : ratio_to_f32_bits(hi, lo, (uint64_t)d_in);
      alpha[row] = __uint_as_float(bits);
    } else {
      partial[2 * (size_t)row] = row_bad ? ~0ull : s_hi;
      partial[2 * (size_t)row + 1] = s_lo;
    }
  }
}

// Per-matrix scale: sum the per-row limbs with 128-bit integers (exact and
// order independent) and round once.
constexpr int kFinalizeThreads = 1024;
constexpr int kFinalizeUnroll = 4;  // rows whose loads are in flight together

__global__ __launch_bounds__(kFinalizeThreads) void compress_finalize_kernel(
    const uint64_t* __restrict__ partial, int d_out, uint64_t n, float* __restrict__ alpha) {
  __shared__ unsigned __int128 s_hi[kFinalizeThreads];
  __shared__ unsigned __int128 s_lo[kFinalizeThreads];
  __shared__ uint32_t s_bad[kFinalizeThreads];
  unsigned __int128 hi = 0, lo = 0;
  uint32_t bad = 0;
  for (int r0 = threadIdx.x; r0 < d_out; r0 += kFinalizeThreads * kFinalizeUnroll) {
    uint64_t h[kFinalizeUnroll], l[kFinalizeUnroll];
#pragma unroll
    for (int u = 0; u < kFinalizeUnroll; ++u) {
      const int r = min(r0 + u * kFinalizeThreads, d_out - 1);
      h[u] = partial[2 * (size_t)r];
      l[u] = partial[2 * (size_t)r + 1];
    }
#pragma unroll
    for (int u = 0; u < kFinalizeUnroll; ++u) {
      if (r0 + u * kFinalizeThreads >= d_out) continue;  // re-read row, not counted
      if (h[u] == ~0ull) {
        bad = 1;
      } else {
        hi += h[u];
      }
      lo += l[u];
    }
  }
  s_hi[threadIdx.x] = hi;
  s_lo[threadIdx.x] = lo;
  s_bad[threadIdx.x] = bad;
  __syncthreads();
  for (int step = kFinalizeThreads / 2; step > 0; step >>= 1) {
    if ((int)threadIdx.x < step) {
      s_hi[threadIdx.x] += s_hi[threadIdx.x + step];
      s_lo[threadIdx.x] += s_lo[threadIdx.x + step];
      s_bad[threadIdx.x] |= s_bad[threadIdx.x + step];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const unsigned __int128 s = (s_hi[0] << 32) + s_lo[0];
    const uint32_t bits =
        s_bad[0] ? 0x7FC00000u : ratio_to_f32_bits((uint64_t)(s >> 64), (uint64_t)s, n);
    alpha[0] = __uint_as_float(bits);
  }
}

}  // namespace

hipError_t launch_compress(const uint16_t* w_ft, const uint16_t* w_base, int d_out, int d_in,
                           int per_row, uint64_t* packed, float* alpha, uint64_t* partial,
                           hipStream_t stream) {
  const dim3 grid((d_out + kRowsPerBlock - 1) / kRowsPerBlock);
  const dim3 block(kRowsPerBlock * kWave);
  if (per_row) {
    hipLaunchKernelGGL(compress_rows_kernel<true>, grid, block, 0, stream, w_ft, w_base, d_out,
                       d_in, packed, alpha, nullptr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(compress_rows_kernel<false>, grid, block, 0, stream, w_ft, w_base, d_out,
                     d_in, packed, nullptr, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compress_finalize_kernel, dim3(1), dim3(kFinalizeThreads), 0, stream,
                     partial, d_out, (uint64_t)d_out * (uint64_t)d_in, alpha);
  return hipGetLastError();
}

}  // namespace bd
