// Calibration kernels: what this GPU actually reaches on a plain stream read
// of HBM and on back-to-back bf16 matrix-core instructions.  They compute
// nothing of the method; the roofline of each library kernel is reported
// against these measured ceilings beside the published peaks.
#include "common.h"
#include "internal.h"
#include "probe.h"

namespace bd {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

// Workgroup b reads bytes [b*chunk, (b+1)*chunk) of src (the last one the
// remainder) with 16-byte loads, four per thread in flight: every wave
// instruction covers a contiguous KiB.  The xor of everything read feeds a
// store that only a chosen value would take, so no load can be dropped.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* src, size_t n16,
                                                                   size_t chunk16,
                                                                   uint32_t* sink) {
  const size_t b0 = (size_t)blockIdx.x * chunk16;
  const size_t b1 = b0 + chunk16 < n16 ? b0 + chunk16 : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = b0 + threadIdx.x;
  constexpr size_t step = (size_t)kProbeThreads * kProbeUnroll;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < b1; i += step) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[i + (size_t)u * kProbeThreads];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (; i < b1; i += kProbeThreads) acc ^= src[i];
  const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == 0x9E3779B9u) sink[blockIdx.x & 255] = r;
}

// Each wave runs eight independent chains of v_mfma_f32_32x32x16_bf16 for
// `iters` steps (8 * iters instructions of 32768 flops each).  The operands
// come from the wave's lane ids so that they are not constants.
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int iters, float* sink) {
  const uint32_t l = threadIdx.x;
  const u32x4 a = {0x3F803F80u ^ (l & 7u), 0x3F003F00u, 0x3E803E80u ^ (l & 3u), 0x3F803F80u};
  const u32x4 b = {0x3F803F80u, 0x3E803E80u ^ (l & 5u), 0x3F003F00u, 0x3F803F80u ^ (l & 1u)};
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mfma32(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (s == 1234.5f) sink[blockIdx.x & 255] = s;
}

// The single-variant decode's loads without its arithmetic, on a 4096 x 4096
// bf16 matrix (256 workgroups of 4 waves, 16 rows each, the 128-element
// blocks of a row round-robin over the waves, each wave starting at block
// (workgroup mod 8) of its range), two blocks of loads in flight per wave:
//   0: contiguous 32 KB per wave instead (1 KB per instruction);
//   1: blocks of 16 consecutive rows x 256 bytes (4 rows per instruction);
//   2: the same with the rows interleaved (chunk k of a workgroup's 4-row
//      chunks = rows 4(b + 256 k) .. +3);
//   3: 2 by buffer loads to LDS;
//   4: 2 plus each block's sign words (4 bytes a lane: 16 rows x 16 bytes);
//   5: 3 plus the sign words plus 1 KB of x a block (the decode ring's loads
//      at up to 4 tokens).
// Register loads are folded by xor into a store that only a chosen value
// takes, so none can be dropped.
constexpr int kDlRowB = 8192;                        // bytes per row
constexpr int kDlMatB = 4096 * kDlRowB;              // 32 MiB
template <int MODE>
__device__ void probe_decode_loads_body(const char* w, const char* signs, const char* x,
                                        uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) char lds[4][8][1024];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wg = blockIdx.x;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(w), (short)0, kDlMatB, 0x00020000);
  u32x4 acc = {0u, 0u, 0u, 0u};
  uint32_t sacc = 0;
  auto row_of = [&](int r) {  // the workgroup's row r (0..15)
    return MODE == 1 ? wg * 16 + r : 4 * (wg + 256 * (r >> 2)) + (r & 3);
  };
  auto blk = [&](int i) { return wv + 4 * ((i + (wg & 7)) & 7); };
  auto off = [&](int t) -> int {  // the wave's t-th weight instruction (0..31)
    if (MODE == 0) return wg * 131072 + wv * 32768 + t * 1024 + lane * 16;
    const int r = 4 * (t & 3) + (lane >> 4);
    return row_of(r) * kDlRowB + blk(t >> 2) * 256 + ((lane & 15) << 4);
  };
  auto sign_word = [&](int i) {  // block i's sign word of lane 4r + j
    return *reinterpret_cast<const uint32_t*>(signs + (size_t)row_of(lane >> 2) * 512 +
                                              blk(i) * 16 + (lane & 3) * 4);
  };
  for (int t0 = 0; t0 < 32; t0 += 8) {
    if (MODE <= 2 || MODE == 4) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off(t0 + u), 0, 0));
      if (MODE == 4) sacc ^= sign_word(t0 >> 2) ^ sign_word((t0 >> 2) + 1);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= v[u];
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (__attribute__((address_space(3))) void*)&lds[wv][u][0], 16, off(t0 + u), 0, 0, 0);
      if (MODE == 5) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc ^= *reinterpret_cast<const u32x4*>(x + blk((t0 >> 2) + h) * 256 + ((lane & 15) << 4));
        sacc ^= sign_word(t0 >> 2) ^ sign_word((t0 >> 2) + 1);
      }
      __builtin_amdgcn_s_waitcnt(0);
      acc ^= *reinterpret_cast<const u32x4*>(&lds[wv][lane & 7][(lane >> 3) * 16]);
    }
  }
  const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3] ^ sacc;
  if (r == 0x9E3779B9u) sink[wg] = r;
}

template <int MODE>
__global__ __launch_bounds__(256) void probe_decode_loads_kernel(const char* w, const char* signs,
                                                                  const char* x, uint32_t* sink) {
  probe_decode_loads_body<MODE>(w, signs, x, sink);
}

}  // namespace

hipError_t launch_probe_decode_loads(const void* w, const void* signs, const void* x, int mode,
                                     uint32_t* sink, hipStream_t stream) {
  const char* cw = static_cast<const char*>(w);
  const char* cs = static_cast<const char*>(signs);
  const char* cx = static_cast<const char*>(x);
  switch (mode) {
    case 0: hipLaunchKernelGGL(probe_decode_loads_kernel<0>, dim3(256), dim3(256), 0, stream, cw, cs, cx, sink); break;
    case 1: hipLaunchKernelGGL(probe_decode_loads_kernel<1>, dim3(256), dim3(256), 0, stream, cw, cs, cx, sink); break;
    case 2: hipLaunchKernelGGL(probe_decode_loads_kernel<2>, dim3(256), dim3(256), 0, stream, cw, cs, cx, sink); break;
    case 3: hipLaunchKernelGGL(probe_decode_loads_kernel<3>, dim3(256), dim3(256), 0, stream, cw, cs, cx, sink); break;
    case 4: hipLaunchKernelGGL(probe_decode_loads_kernel<4>, dim3(256), dim3(256), 0, stream, cw, cs, cx, sink); break;
    case 5: hipLaunchKernelGGL(probe_decode_loads_kernel<5>, dim3(256), dim3(256), 0, stream, cw, cs, cx, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, size_t bytes, int workgroups, uint32_t* sink,
                             hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const size_t chunk16 = (n16 + (size_t)workgroups - 1) / (size_t)workgroups;
  hipLaunchKernelGGL(probe_read_kernel, dim3(workgroups), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(src), n16, chunk16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int workgroups, int iters, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(workgroups), dim3(kProbeThreads), 0, stream, iters,
                     sink);
  return hipGetLastError();
}

}  // namespace bd
