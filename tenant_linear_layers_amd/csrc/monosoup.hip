// MonoSoup merge on gfx950: k fine-tuned checkpoints of one base merged
// through rank-r truncations of their task vectors.
//
// Page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak", section
// "MonoSoup": each Delta_i = W_i - W_base is replaced by its rank-r truncated
// SVD tau_i, and W_merged = W_base + (1/k) sum_i tau_i.
//
// tau_i is the projection of Delta_i onto its top-r left singular subspace,
// tau_i = Q_i Q_i^T Delta_i for Q_i with orthonormal columns spanning that
// subspace.  Q_i comes from orthogonal (subspace) iteration started from a
// caller-drawn Gaussian Omega [d_in, r]: Y = Delta Omega, then q times
// Y <- Delta (Delta^T Y), each product re-orthonormalised (CholeskyQR; twice
// for the final basis).
// It converges to the top-r subspace when sigma_r > sigma_{r+1}, with error
// falling like (sigma_{r+1} / sigma_r)^(2q+1) times a factor from the random
// start (growing like sqrt(r (d_out - r))); then Z_i = Delta_i^T Q_i and
// tau_i = Q_i Z_i^T.  No small SVD is needed.
//
// Every product streams Delta straight from the two bf16 matrices (one
// float32 subtraction per element, like the compression); all sums run in
// float32 in a fixed order (deterministic).  The working width R is the rank
// rounded up to 8, 16 or 32; columns past the rank start as zeros and stay
// zero (their Cholesky pivots are dropped).
//
// Kernels: mul (Y = Delta X: 8 rows per wave (4 at width 32), lanes across d_in, a
// butterfly sum per output), tmul (partial Z = Delta^T Y over row chunks,
// lanes across d_in) and its fixed-order reduction, gram (partial A^T A over
// row chunks), chol (sum of the partials and the Cholesky factor with
// dropped pivots, one workgroup), scale (A <- A U^-1 by substitution, one row
// per thread), merge (W_base + mean of Q_i Z_i^T, rounded to bf16, LDS
// tiles).
#include "common.h"
#include "internal.h"

namespace bd {
namespace {

constexpr int kTmulChunks = 64;   // row chunks of the Delta^T Y partials
constexpr int kGramChunks = 64;   // row chunks of the Gram partials

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Delta of 8 consecutive elements from two 16-byte bf16 loads.
__device__ __forceinline__ void delta8(const u32x4& a, const u32x4& b, float (&d)[8]) {
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    d[2 * h] = bf16_lo(a[h]) - bf16_lo(b[h]);
    d[2 * h + 1] = bf16_hi(a[h]) - bf16_hi(b[h]);
  }
}

// Y[o][j] = sum_c Delta[o][c] X[c][j]; X [d_in][R], Y [d_out][R].  A wave
// owns RW rows, which share every read of X; one wave per workgroup.
template <int R, int RW>
__global__ __launch_bounds__(64) void ms_mul_kernel(const uint16_t* __restrict__ wf,
                                                    const uint16_t* __restrict__ wb, int d_out,
                                                    int d_in, const float* __restrict__ X,
                                                    float* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int o0 = blockIdx.x * RW;
  float acc[RW][R];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j) acc[i][j] = 0.f;
  for (int c0 = lane * 8; c0 < d_in; c0 += 512) {
    float d[RW][8];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const size_t base = (size_t)min(o0 + i, d_out - 1) * d_in + c0;
      delta8(ld128(wf + base), ld128(wb + base), d[i]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float* xr = X + (size_t)(c0 + e) * R;
#pragma unroll
      for (int j4 = 0; j4 < R / 4; ++j4) {
        const float4 x = *reinterpret_cast<const float4*>(xr + 4 * j4);
#pragma unroll
        for (int i = 0; i < RW; ++i) {
          acc[i][4 * j4] += d[i][e] * x.x;
          acc[i][4 * j4 + 1] += d[i][e] * x.y;
          acc[i][4 * j4 + 2] += d[i][e] * x.z;
          acc[i][4 * j4 + 3] += d[i][e] * x.w;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float v = acc[i][j];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
      acc[i][j] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      if (o0 + i >= d_out) continue;
#pragma unroll
      for (int j = 0; j < R; ++j) Y[(size_t)(o0 + i) * R + j] = acc[i][j];
    }
  }
}

// Zp[p][c][j] = sum over rows o of chunk p of Delta[o][c] Y[o][j]; one wave
// per (128-column block, chunk), two columns per lane.
template <int R>
__global__ __launch_bounds__(64) void ms_tmul_kernel(const uint16_t* __restrict__ wf,
                                                     const uint16_t* __restrict__ wb, int d_out,
                                                     int d_in, const float* __restrict__ Y,
                                                     float* __restrict__ Zp) {
  const int lane = threadIdx.x;
  const int c = blockIdx.x * 128 + 2 * lane;
  const bool live = c < d_in;
  const int cc = live ? c : d_in - 2;
  const int p = blockIdx.y;
  const int rows = (d_out + kTmulChunks - 1) / kTmulChunks;
  const int r0 = p * rows;
  const int r1 = min(r0 + rows, d_out);
  float acc[2][R];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < R; ++j) acc[h][j] = 0.f;
#pragma unroll 4
  for (int o = r0; o < r1; ++o) {
    const size_t base = (size_t)o * d_in + cc;
    const uint32_t a = ld32(wf + base);
    const uint32_t b = ld32(wb + base);
    const float d0 = bf16_lo(a) - bf16_lo(b);
    const float d1 = bf16_hi(a) - bf16_hi(b);
    const float* yr = Y + (size_t)o * R;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float y = yr[j];
      acc[0][j] += d0 * y;
      acc[1][j] += d1 * y;
    }
  }
  if (live) {
    float* z = Zp + ((size_t)p * d_in + c) * R;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j4 = 0; j4 < R / 4; ++j4)
        *reinterpret_cast<float4*>(z + h * R + 4 * j4) =
            make_float4(acc[h][4 * j4], acc[h][4 * j4 + 1], acc[h][4 * j4 + 2], acc[h][4 * j4 + 3]);
  }
}

// Z[i] = sum_p Zp[p][i] in chunk order (n = d_in * R values).
__global__ __launch_bounds__(256) void ms_reduce_kernel(const float* __restrict__ Zp, int64_t n,
                                                        float* __restrict__ Z) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
#pragma unroll 16
  for (int p = 0; p < kTmulChunks; ++p) s += Zp[(int64_t)p * n + i];
  Z[i] = s;
}

// Gp[p][a][b] = sum over rows of chunk p of A[row][a] A[row][b]; A [n][R].
template <int R>
__global__ __launch_bounds__(R * R) void ms_gram_kernel(const float* __restrict__ A, int n,
                                                        float* __restrict__ Gp) {
  const int a = threadIdx.x / R;
  const int b = threadIdx.x % R;
  const int p = blockIdx.x;
  const int rows = (n + kGramChunks - 1) / kGramChunks;
  const int r0 = p * rows;
  const int r1 = min(r0 + rows, n);
  float s = 0.f;
#pragma unroll 8
  for (int o = r0; o < r1; ++o) s += A[(size_t)o * R + a] * A[(size_t)o * R + b];
  Gp[((size_t)p * R + a) * R + b] = s;
}

// G = sum_p Gp[p] (chunk order) and its upper Cholesky factor U (G = U^T U),
// written to Uf [R][R].  Thread (a, b) keeps G[a][b] (b >= a) in a register
// and the factorisation runs one pivot per step: the step's row of U from the
// updated row of G, then the trailing update.  A pivot at or below 1e-6 of
// the largest diagonal of G is dropped: its row of U is zero, its diagonal
// 0 marks it for the substitution.
template <int R>
__global__ __launch_bounds__(R * R) void ms_chol_kernel(const float* __restrict__ Gp,
                                                        float* __restrict__ Uf) {
  __shared__ float U[R][R];
  __shared__ float diag[R];
  __shared__ float piv;
  const int a = threadIdx.x / R;
  const int b = threadIdx.x % R;
  float g = 0.f;
#pragma unroll
  for (int p = 0; p < kGramChunks; ++p) g += Gp[((size_t)p * R + a) * R + b];
  U[a][b] = 0.f;
  if (a == b) diag[a] = g;
  __syncthreads();
  float gmax = 0.f;
  for (int k = 0; k < R; ++k) gmax = fmaxf(gmax, diag[k]);
  const float thr = 1e-6f * gmax;
  for (int k = 0; k < R; ++k) {
    if (a == k && b == k) piv = g;
    __syncthreads();
    const float pk = piv;
    const bool keep = gmax > 0.f && pk > thr;
    if (a == k && b >= k) U[k][b] = keep ? g / sqrtf(pk) : 0.f;
    __syncthreads();
    if (a > k && b >= a) g -= U[k][a] * U[k][b];
  }
  Uf[a * R + b] = U[a][b];
}

// A[row][:] <- A[row][:] U^-1 on the kept indices, by forward substitution
// (z U = x, z_j = 0 where U[j][j] = 0); one row per thread.
template <int R>
__global__ __launch_bounds__(256) void ms_scale_kernel(float* __restrict__ A, int n,
                                                       const float* __restrict__ Uf) {
  __shared__ float M[R * R];
  for (int t = threadIdx.x; t < R * R; t += 256) M[t] = Uf[t];
  __syncthreads();
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= n) return;
  float z[R];
#pragma unroll
  for (int j = 0; j < R; ++j) z[j] = A[(size_t)row * R + j];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    float v = z[j];
#pragma unroll
    for (int m = 0; m < j; ++m) v -= z[m] * M[m * R + j];
    const float ujj = M[j * R + j];
    z[j] = ujj > 0.f ? v / ujj : 0.f;
  }
#pragma unroll
  for (int j = 0; j < R; ++j) A[(size_t)row * R + j] = z[j];
}

// Omega [d_in][rank] into X [d_in][R], zero columns past the rank.
__global__ __launch_bounds__(256) void ms_pad_kernel(const float* __restrict__ omega, int d_in,
                                                     int rank, int R, float* __restrict__ X) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)d_in * R) return;
  const int c = (int)(i / R);
  const int j = (int)(i % R);
  X[i] = j < rank ? omega[(size_t)c * rank + j] : 0.f;
}

// out[o][c] = bf16(W_base[o][c] + (1/k) sum_i sum_j Y_i[o][j] Z_i[c][j]);
// tau (optional) the float32 mean.  A workgroup owns 16 rows x 128 columns;
// thread t takes row t/16 and columns 8*(t%16) .. +7; each checkpoint's Y
// rows and Z columns of the tile go through LDS.
template <int R>
__global__ __launch_bounds__(256) void ms_merge_kernel(const uint16_t* __restrict__ wb, int d_out,
                                                       int d_in, int k, const float* __restrict__ Y,
                                                       const float* __restrict__ Z,
                                                       uint16_t* __restrict__ out,
                                                       float* __restrict__ tau) {
  __shared__ float Ys[16][R];
  __shared__ __attribute__((aligned(16))) float Zs[R][128];  // transposed: a thread's 8
                                                              // columns are 32 contiguous bytes
  const int t = threadIdx.x;
  const int o0 = blockIdx.y * 16;
  const int c0 = blockIdx.x * 128;
  const int lr = t >> 4;
  const int lc = (t & 15) * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int i = 0; i < k; ++i) {
    const float* Yi = Y + (size_t)i * d_out * R;
    const float* Zi = Z + (size_t)i * d_in * R;
    __syncthreads();
    for (int u = t; u < 16 * R; u += 256) {
      const int r = u / R, j = u % R;
      Ys[r][j] = Yi[(size_t)min(o0 + r, d_out - 1) * R + j];
    }
    for (int u = t; u < 128 * R; u += 256) {
      const int cc = u / R, j = u % R;
      Zs[j][cc] = Zi[(size_t)min(c0 + cc, d_in - 1) * R + j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float y = Ys[lr][j];
      const float4 z0 = *reinterpret_cast<const float4*>(&Zs[j][lc]);
      const float4 z1 = *reinterpret_cast<const float4*>(&Zs[j][lc + 4]);
      acc[0] += y * z0.x;
      acc[1] += y * z0.y;
      acc[2] += y * z0.z;
      acc[3] += y * z0.w;
      acc[4] += y * z1.x;
      acc[5] += y * z1.y;
      acc[6] += y * z1.z;
      acc[7] += y * z1.w;
    }
  }
  const int o = o0 + lr;
  const int c = c0 + lc;
  if (o >= d_out || c >= d_in) return;
  const float invk = 1.f / (float)k;
  const size_t base = (size_t)o * d_in + c;
  const u32x4 w = ld128(wb + base);
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float t0 = acc[2 * h] * invk;
    const float t1 = acc[2 * h + 1] * invk;
    r[h] = (uint32_t)f32_to_bf16_bits(bf16_lo(w[h]) + t0) |
           ((uint32_t)f32_to_bf16_bits(bf16_hi(w[h]) + t1) << 16);
    if (tau) {
      tau[base + 2 * h] = t0;
      tau[base + 2 * h + 1] = t1;
    }
  }
  *reinterpret_cast<u32x4*>(out + base) = r;
}

template <int R>
struct Plan {
  int d_out, d_in, k;
  float *Y, *Z, *X0, *Zp, *Gp, *Uf;
  hipStream_t s;

  // passes = 2 (CholeskyQR2) for the final basis; inside the iteration one
  // pass is enough, since every step re-orthonormalises what it multiplies.
  hipError_t orth(float* A, int n, int passes) const {
    for (int pass = 0; pass < passes; ++pass) {
      hipLaunchKernelGGL(ms_gram_kernel<R>, dim3(kGramChunks), dim3(R * R), 0, s, A, n, Gp);
      hipLaunchKernelGGL(ms_chol_kernel<R>, dim3(1), dim3(R * R), 0, s, Gp, Uf);
      hipLaunchKernelGGL(ms_scale_kernel<R>, dim3((n + 255) / 256), dim3(256), 0, s, A, n, Uf);
    }
    return hipGetLastError();
  }
  hipError_t mul(const uint16_t* wf, const uint16_t* wb, const float* X, float* Yo) const {
    constexpr int RW = R <= 16 ? 8 : 4;
    hipLaunchKernelGGL((ms_mul_kernel<R, RW>), dim3((d_out + RW - 1) / RW), dim3(64), 0, s, wf, wb,
                       d_out, d_in, X, Yo);
    return hipGetLastError();
  }
  hipError_t tmul(const uint16_t* wf, const uint16_t* wb, const float* Yi, float* Zo) const {
    hipLaunchKernelGGL(ms_tmul_kernel<R>, dim3((d_in + 127) / 128, kTmulChunks), dim3(64), 0, s,
                       wf, wb, d_out, d_in, Yi, Zp);
    const int64_t n = (int64_t)d_in * R;
    hipLaunchKernelGGL(ms_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, Zp,
                       n, Zo);
    return hipGetLastError();
  }
};

template <int R>
hipError_t run_monosoup(const uint16_t* const* w_ft, int k, const uint16_t* w_base, int d_out,
                        int d_in, int rank, int q, const float* omega, uint16_t* out, float* tau,
                        char* ws, hipStream_t s) {
  Plan<R> P;
  P.d_out = d_out;
  P.d_in = d_in;
  P.k = k;
  P.s = s;
  const size_t nY = (size_t)k * d_out * R, nZ = (size_t)k * d_in * R;
  float* f = reinterpret_cast<float*>(ws);
  P.Y = f;
  P.Z = P.Y + nY;
  P.X0 = P.Z + nZ;
  P.Zp = P.X0 + (size_t)d_in * R;
  P.Gp = P.Zp + (size_t)kTmulChunks * d_in * R;
  P.Uf = P.Gp + (size_t)kGramChunks * R * R;
  hipLaunchKernelGGL(ms_pad_kernel, dim3((unsigned)(((size_t)d_in * R + 255) / 256)), dim3(256), 0,
                     s, omega, d_in, rank, R, P.X0);
  hipError_t e = hipGetLastError();
  for (int i = 0; i < k && e == hipSuccess; ++i) {
    float* Yi = P.Y + (size_t)i * d_out * R;
    float* Zi = P.Z + (size_t)i * d_in * R;
    e = P.mul(w_ft[i], w_base, P.X0, Yi);
    if (e == hipSuccess) e = P.orth(Yi, d_out, q == 0 ? 2 : 1);
    for (int it = 0; it < q && e == hipSuccess; ++it) {
      e = P.tmul(w_ft[i], w_base, Yi, Zi);
      if (e == hipSuccess) e = P.orth(Zi, d_in, 1);
      if (e == hipSuccess) e = P.mul(w_ft[i], w_base, Zi, Yi);
      if (e == hipSuccess) e = P.orth(Yi, d_out, it == q - 1 ? 2 : 1);
    }
    if (e == hipSuccess) e = P.tmul(w_ft[i], w_base, Yi, Zi);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ms_merge_kernel<R>, dim3((d_in + 127) / 128, (d_out + 15) / 16), dim3(256),
                     0, s, w_base, d_out, d_in, k, P.Y, P.Z, out, tau);
  return hipGetLastError();
}

}  // namespace

int monosoup_width(int rank) { return rank <= 8 ? 8 : (rank <= 16 ? 16 : 32); }

size_t monosoup_workspace_bytes(int64_t d_out, int64_t d_in, int k, int rank) {
  const int64_t R = monosoup_width(rank);
  return 4u * (size_t)(k * d_out * R + k * d_in * R + d_in * R + (int64_t)kTmulChunks * d_in * R +
                       (int64_t)kGramChunks * R * R + R * R);
}

hipError_t launch_monosoup(const uint16_t* const* w_ft, int k, const uint16_t* w_base, int d_out,
                           int d_in, int rank, int power_iters, const float* omega, uint16_t* out,
                           float* tau, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  switch (monosoup_width(rank)) {
    case 8:
      return run_monosoup<8>(w_ft, k, w_base, d_out, d_in, rank, power_iters, omega, out, tau, ws,
                             stream);
    case 16:
      return run_monosoup<16>(w_ft, k, w_base, d_out, d_in, rank, power_iters, omega, out, tau, ws,
                              stream);
    default:
      return run_monosoup<32>(w_ft, k, w_base, d_out, d_in, rank, power_iters, omega, out, tau, ws,
                              stream);
  }
}

}  // namespace bd
