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
// CholeskyQR of A is Q = A U^+ with U the Cholesky factor of A^T A and U^+
// the inverse on the kept pivots (zero rows and columns for dropped ones).
// The products are linear, so Delta (A U^+) = (Delta A) U^+: the scaling of
// one basis is applied to the next product's output rows instead of being a
// pass of its own, and the stored A is the unscaled product.
//
// Kernels, two per product:
//   mul / tmul   Y = Delta X and Z = Delta^T Y on the matrix cores
//                (v_mfma_f32_16x16x4_f32), Delta formed in registers from
//                16-byte loads of both matrices; four waves per workgroup
//                split the contraction and add through LDS; the workgroups
//                along the contraction write partial sums.  One extra
//                workgroup meanwhile factors the Gram matrix of the
//                previous product (its partials summed in order, Cholesky
//                with dropped pivots, U^+), which only the next epilogue
//                needs.
//   epi          sums the partials in order, multiplies by the previous
//                U^+, writes the rows and a Gram partial per 64 rows.  The
//                same kernel in place scales a basis (with or without its
//                Gram partials).
//   factor       the Gram factorisation on its own, where no product follows.
//   merge        W_base + (1/k) sum_i Q_i Z_i^T, an fp32 matrix-core product
//                with K = k R, rounded to bf16 through an LDS tile.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace bd {
namespace {

constexpr int kWaves = 4;     // waves per workgroup of the products
constexpr int kEpiRows = 64;  // rows per workgroup of the epilogue

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

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// A Gram factorisation for the extra workgroup of a product kernel (none when
// Gp is null): Mout = U^+ from the nb partials at Gp.
struct FactorJob {
  const float* Gp;
  int nb;
  float* Mout;
};

// Workgroups along the contraction of mul: about 512 workgroups in all, each
// wave at least one 32-column block, at most 32.
inline int ms_mul_slices(int64_t d_out, int64_t d_in) {
  const int64_t groups = (d_out + 63) / 64;
  int64_t ks = (512 + groups - 1) / groups;
  const int64_t most = d_in / 32 / kWaves;
  ks = ks > most ? most : ks;
  ks = ks > 32 ? 32 : ks;
  return (int)(ks < 1 ? 1 : ks);
}

// Row chunks of tmul: about 512 workgroups, at least 32 rows each, at most 32.
inline int ms_tmul_chunks(int64_t d_out, int64_t d_in) {
  const int64_t groups = (d_in + 127) / 128;
  int64_t kt = (512 + groups - 1) / groups;
  const int64_t most = (d_out + 31) / 32;
  kt = kt > most ? most : kt;
  kt = kt > 32 ? 32 : kt;
  return (int)(kt < 1 ? 1 : kt);
}

// LDS floats that gram_factor needs.
template <int R>
constexpr int factor_smem() {
  return 1024 + 2 * R * R + 4;
}

// G = the sum of the nb Gram partials Gp[0 .. nb-1] in order, its Cholesky
// factor U with dropped pivots (a pivot at or below 1e-6 of the largest
// diagonal of G: its row of U is zero) and Mout = U^+, the upper-triangular
// matrix with z = x U^+ solving z U = x on the kept indices (z zero on the
// dropped ones).  One workgroup of 256 threads; sm: factor_smem<R>() floats
// of LDS, 16-byte aligned.
template <int R>
__device__ void gram_factor(const float* __restrict__ Gp, int nb, float* __restrict__ Mout,
                            float* sm) {
  float4* S4 = reinterpret_cast<float4*>(sm);
  float(*G)[R] = reinterpret_cast<float(*)[R]>(sm + 1024);
  float(*U)[R] = reinterpret_cast<float(*)[R]>(sm + 1024 + R * R);
  float& piv = sm[1024 + 2 * R * R];
  const int t = threadIdx.x;
  // G = sum of the partials in workgroup order: thread t adds float4 q of
  // partials h, h + H, ... (q = t % F, h = t / F); then the H sums in h order
  constexpr int F = R * R / 4;
  constexpr int H = 256 / F;
  {
    const int q = t % F, h = t / F;
    const float* src = Gp + 4 * q;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    int b = h;
    // eight loads in flight, then their sums in order
    for (; b + 7 * H < nb; b += 8 * H) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const float4*>(src + (size_t)(b + u * H) * R * R);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s.x += v[u].x;
        s.y += v[u].y;
        s.z += v[u].z;
        s.w += v[u].w;
      }
    }
    for (; b < nb; b += H) {
      const float4 v = *reinterpret_cast<const float4*>(src + (size_t)b * R * R);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    S4[t] = s;
  }
  __syncthreads();
  if (t < F) {
    float4 s = S4[t];
    for (int h = 1; h < H; ++h) {
      const float4 v = S4[h * F + t];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    float* gr = &G[0][0] + 4 * t;
    gr[0] = s.x;
    gr[1] = s.y;
    gr[2] = s.z;
    gr[3] = s.w;
  }
  __syncthreads();
  // Cholesky with dropped pivots: thread t keeps G entries t, t + 256, ...
  constexpr int NE = (R * R + 255) / 256;
  float gv[NE];
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const int e = t + 256 * u;
    gv[u] = e < R * R ? G[e / R][e % R] : 0.f;
    if (e < R * R) U[e / R][e % R] = 0.f;
  }
  float gmax = 0.f;
  for (int kk = 0; kk < R; ++kk) gmax = fmaxf(gmax, G[kk][kk]);
  const float thr = 1e-6f * gmax;
  __syncthreads();
  for (int kk = 0; kk < R; ++kk) {
#pragma unroll
    for (int u = 0; u < NE; ++u)
      if (t + 256 * u == kk * R + kk) piv = gv[u];
    __syncthreads();
    const float pk = piv;
    const bool keep = gmax > 0.f && pk > thr;
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = t + 256 * u, a = e / R, b = e % R;
      if (e < R * R && a == kk && b >= kk) U[kk][b] = keep ? gv[u] / sqrtf(pk) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = t + 256 * u, a = e / R, b = e % R;
      if (e < R * R && a > kk && b >= a) gv[u] -= U[kk][a] * U[kk][b];
    }
  }
  // row m of U^+ is the substitution of the unit vector e_m (thread m)
  if (t < R) {
    float z[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float v = j == t ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < j; ++m) v -= z[m] * U[m][j];
      const float ujj = U[j][j];
      z[j] = ujj > 0.f ? v / ujj : 0.f;
    }
#pragma unroll
    for (int j = 0; j < R; ++j) Mout[t * R + j] = z[j];
  }
}

// Position of 16-byte chunk c of a staged 64-byte row r: the operand reads
// of 16 consecutive rows at one chunk hit distinct banks whether the LDS
// serves 8 or 16 lanes of a 16-byte read per cycle.
__device__ __forceinline__ int ms_swz(int r, int c) {
  return c ^ (((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1));
}

// Yp[ks][o][j] = sum over the workgroup's columns c of Delta[o][c] X[c][j];
// X [d_in][R].  A workgroup owns 64 rows (four 16-row tiles) and the 32-wide
// column blocks 4 ks + w, 4 ks + w + 4 KS, ... for wave w.  Each wave stages
// its block of both bf16 matrices (64 rows x 64 bytes each) by buffer loads
// to LDS, four lanes per row (every quad of lanes one contiguous 64-byte
// piece, which the address unit serves about four times faster than loads
// in the operand layout), one block ahead in a ring of two stages; X's rows
// of the block go to registers with it.  Lane (n, g) then reads columns
// 8g .. 8g+7 of row n of each tile and holds X's rows 8g .. 8g+7 for column
// n of each 16-column tile; product s takes the block's columns s, 8+s,
// 16+s, 24+s.  The waves' sums are added through LDS in wave order.
template <int R>
__global__ __launch_bounds__(256) void ms_mul_kernel(const uint16_t* __restrict__ wf,
                                                     const uint16_t* __restrict__ wb, int d_out,
                                                     int d_in, int KS, const float* __restrict__ X,
                                                     float* __restrict__ Yp, FactorJob fj) {
  constexpr int NC = (R + 15) / 16;         // 16-column tiles of X and Y
  constexpr int E = 4 * NC * 4;             // accumulator floats per lane
  constexpr int kWaveStage = 2 * 64 * 64;   // a wave's block of both matrices
  constexpr int kStage = kWaves * kWaveStage;
  constexpr int kLoads = 8 + 8 * NC;        // vector loads per block
  static_assert(kWaves * E * 64 * 4 <= kStage && factor_smem<R>() * 4 <= kStage,
                "the reduction and the factorisation fit in the first stage");
  static_assert(kLoads < 64, "vmcnt holds 6 bits");
  // one array per stage: the compiler's wait insertion tells separate LDS
  // arrays apart, so reads of one stage do not wait for loads into the other
  __shared__ __attribute__((aligned(16))) char st0[kStage];
  __shared__ __attribute__((aligned(16))) char st1[kStage];
  float* sm = reinterpret_cast<float*>(st0);
  // the extra workgroup after the row groups (its index from d_out, not
  // gridDim: a read of the dispatch packet would delay every first load)
  if (blockIdx.x == (unsigned)((d_out + 63) >> 6) && fj.Gp) {
    if (blockIdx.y == 0) gram_factor<R>(fj.Gp, fj.nb, fj.Mout, sm);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int n = lane & 15;
  const int g = lane >> 4;
  const int row0 = blockIdx.x * 64;
  const int ks = blockIdx.y;
  const int nblk = d_in >> 5;
  // rows past d_out lie beyond the buffers and read as zero
  const int nbytes = min(64, d_out - row0) * d_in * 2;
  const uint16_t* fblk = wf + (size_t)row0 * d_in;
  const uint16_t* bblk = wb + (size_t)row0 * d_in;
  // staging instruction j: rows 16j .. 16j+15, lane l row 16j + l/4 at
  // position l%4 (global chunk ms_swz(row, l%4)); operand reads of tile t:
  // row 16t + n, chunk g
  int voff[4], roff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 16 * j + (lane >> 2);
    voff[j] = r * d_in * 2 + (ms_swz(r, lane & 3) << 4);
    const int rr = 16 * j + n;
    roff[j] = rr * 64 + (ms_swz(rr, g) << 4);
  }
  const int kb0 = ks * kWaves + w;
  const int kstep = KS * kWaves;
  const int nmine = kb0 < nblk ? (nblk - 1 - kb0) / kstep + 1 : 0;

  f32x4 acc[4][NC];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) acc[t][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float xv[2][NC][8];
  auto issue = [&](int i, int su) {
    const int c0 = (kb0 + i * kstep) << 5;
    char* st = (su == 0 ? st0 : st1) + w * kWaveStage;
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_bload16(fblk, nbytes, voff[j], c0 * 2, st + j * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_bload16(bblk, nbytes, voff[j], c0 * 2, st + 4096 + j * 1024);
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      const float* xc = X + (size_t)(c0 + 8 * g) * R + min(16 * ct + n, R - 1);
#pragma unroll
      for (int s = 0; s < 8; ++s) xv[su][ct][s] = xc[(size_t)s * R];
    }
  };
  if (nmine > 0) issue(0, 0);
  for (int i0 = 0; i0 < nmine; i0 += 2) {
#pragma unroll
    for (int su = 0; su < 2; ++su) {
      const int i = i0 + su;
      // the stage about to be refilled was read by the previous block: its
      // LDS reads complete before the buffer loads may write it, and the
      // loads stay below this point
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      // past the wave's last block the issue re-reads that block into the
      // stage nobody reads: every block issues the same number of loads
      issue(min(i + 1, nmine - 1), su ^ 1);
      __builtin_amdgcn_sched_barrier(0);  // the next block's loads stay together, here
      __builtin_amdgcn_s_waitcnt((kLoads & 15) | ((kLoads >> 4) << 14) | (0x7 << 4) |
                                 (0xF << 8));  // vmcnt only: block i is in
      // No branch on i: past the wave's last block X is taken as zero (the
      // stage holds a re-read of that block), which adds nothing; with a
      // branch the compiler moves the next block's loads into it.
      const bool live = i < nmine;
      const char* st = (su == 0 ? st0 : st1) + w * kWaveStage;
      float d[4][8];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        delta8(*reinterpret_cast<const u32x4*>(st + roff[t]),
               *reinterpret_cast<const u32x4*>(st + 4096 + roff[t]), d[t]);
      float xm[NC][8];
#pragma unroll
      for (int ct = 0; ct < NC; ++ct)
#pragma unroll
        for (int s = 0; s < 8; ++s) xm[ct][s] = live && 16 * ct + n < R ? xv[su][ct][s] : 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int ct = 0; ct < NC; ++ct) acc[t][ct] = mfma_f32(d[t][s], xm[ct][s], acc[t][ct]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the last re-reads have landed
  __syncthreads();                // the first stage becomes the reduction area
  float(*red)[E][64] = reinterpret_cast<float(*)[E][64]>(sm);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int ct = 0; ct < NC; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[w][(t * NC + ct) * 4 + v][lane] = acc[t][ct][v];
  __syncthreads();
  // wave w adds the waves' sums of groups (t, ct) = w, w + 4, ...; the
  // 16x16 output layout puts rows 4g .. 4g+3 of column n in lane (n, g)
  for (int q = w; q < 4 * NC; q += kWaves) {
    const int t = q / NC, ct = q % NC;
    const int j = 16 * ct + n;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int idx = q * 4 + v;
      const float sum =
          ((red[0][idx][lane] + red[1][idx][lane]) + red[2][idx][lane]) + red[3][idx][lane];
      const int row = row0 + 16 * t + 4 * g + v;
      if (row < d_out && j < R) Yp[((size_t)ks * d_out + row) * R + j] = sum;
    }
  }
}

// Zp[p][c][j] = sum over rows o of chunk p of Delta[o][c] Y[o][j], as
// Z^T = Y^T Delta.  A workgroup owns 128 columns and one row chunk; wave w
// takes the 8-row steps w, w + 4, ... of the chunk.  Per 4-row step lane
// (n, g) holds Y[o+g][16ct+n] (operand A) and columns 8n .. 8n+7 of row o+g
// (one 16-byte load of each bf16 matrix); product e takes column 8n+e of
// every lane, so accumulator (e, ct) of lane (n, g) ends with
// Z[8n+e][16ct+4g+v], v = 0..3.  The waves' sums are added through LDS.
template <int R>
__global__ __launch_bounds__(256) void ms_tmul_kernel(const uint16_t* __restrict__ wf,
                                                      const uint16_t* __restrict__ wb, int d_out,
                                                      int d_in, int KT, const float* __restrict__ Y,
                                                      float* __restrict__ Zp, FactorJob fj) {
  constexpr int NC = (R + 15) / 16;
  constexpr int E = 8 * NC * 4;
  constexpr int NS = std::max(kWaves * E * 64, factor_smem<R>());
  __shared__ __attribute__((aligned(16))) float sm[NS];
  if (blockIdx.x == (unsigned)((d_in + 127) >> 7) && fj.Gp) {  // the extra workgroup
    if (blockIdx.y == 0) gram_factor<R>(fj.Gp, fj.nb, fj.Mout, sm);
    return;
  }
  float(*red)[E][64] = reinterpret_cast<float(*)[E][64]>(sm);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int c = blockIdx.x * 128 + 8 * n;
  const bool live = c < d_in;
  const int cc = live ? c : 0;
  const int p = blockIdx.y;
  const int rows = ((d_out + KT - 1) / KT + 31) & ~31;
  const int r0 = p * rows;
  const int r1 = min(r0 + rows, d_out);
  f32x4 acc[8][NC];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) acc[e][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  // two 4-row steps per pass with their loads first (the products are
  // convergent operations, which the compiler does not unroll by a runtime
  // trip count)
  for (int o0 = r0 + 8 * w; o0 < r1; o0 += 8 * kWaves) {
    float d[2][8], y[2][NC];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int o = o0 + 4 * h + g;
      const int oc = min(o, d_out - 1);
      const size_t base = (size_t)oc * d_in + cc;
      delta8(ld128(wf + base), ld128(wb + base), d[h]);
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const int j = 16 * ct + n;
        const float v = Y[(size_t)oc * R + min(j, R - 1)];
        y[h][ct] = o < r1 && j < R ? v : 0.f;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int ct = 0; ct < NC; ++ct) acc[e][ct] = mfma_f32(y[h][ct], d[h][e], acc[e][ct]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int ct = 0; ct < NC; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[w][(e * NC + ct) * 4 + v][lane] = acc[e][ct][v];
  __syncthreads();
  if (!live) return;
  for (int q = w; q < 8 * NC; q += kWaves) {
    const int e = q / NC, ct = q % NC;
    const int j = 16 * ct + 4 * g;
    float s[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int idx = q * 4 + v;
      s[v] = ((red[0][idx][lane] + red[1][idx][lane]) + red[2][idx][lane]) + red[3][idx][lane];
    }
    if (j < R)
      *reinterpret_cast<float4*>(Zp + ((size_t)p * d_in + c + e) * R + j) =
          make_float4(s[0], s[1], s[2], s[3]);
  }
}

// The epilogue of a product, and the in-place scaling of a basis:
//   A[row] = (sum_p P[p][row]) Min        (Min = identity when null)
// over 64-row tiles, one per workgroup; with Gp, each workgroup also writes
// the Gram partial of its rows, A_tile^T A_tile, to Gp[workgroup].  P may
// alias A (parts = 1): every workgroup reads its whole tile before writing.
template <int R>
__global__ __launch_bounds__(256) void ms_epi_kernel(const float* P, int parts, int n,
                                                     const float* __restrict__ Min, float* A,
                                                     float* __restrict__ Gp) {
  constexpr int RB = kEpiRows;
  constexpr int Q4 = R / 4;    // float4 per row
  constexpr int V4 = RB * Q4;  // float4 per tile
  __shared__ float T[RB][R + 1];
  __shared__ float Zs[RB][R + 1];
  __shared__ float Ms[R][R];
  const int t = threadIdx.x;
  const int row0 = blockIdx.x * RB;
  const size_t plane = (size_t)n * R;
  for (int f = t; f < V4; f += 256) {
    const int r = f / Q4, j = 4 * (f % Q4);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row0 + r < n) {
      const float* src = P + (size_t)(row0 + r) * R + j;
#pragma unroll 4
      for (int p = 0; p < parts; ++p) {
        const float4 v = *reinterpret_cast<const float4*>(src + p * plane);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
      }
    }
    T[r][j] = s.x;
    T[r][j + 1] = s.y;
    T[r][j + 2] = s.z;
    T[r][j + 3] = s.w;
  }
  if (Min)
    for (int e = t; e < R * R; e += 256) Ms[e / R][e % R] = Min[e];
  __syncthreads();
  for (int f = t; f < V4; f += 256) {
    const int r = f / Q4, j = 4 * (f % Q4);
    float z[4];
    if (Min) {
#pragma unroll
      for (int u = 0; u < 4; ++u) z[u] = 0.f;
#pragma unroll
      for (int m = 0; m < R; ++m) {
        const float x = T[r][m];
#pragma unroll
        for (int u = 0; u < 4; ++u) z[u] += x * Ms[m][j + u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) z[u] = T[r][j + u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) Zs[r][j + u] = z[u];
    if (row0 + r < n)
      *reinterpret_cast<float4*>(A + (size_t)(row0 + r) * R + j) =
          make_float4(z[0], z[1], z[2], z[3]);
  }
  if (!Gp) return;
  __syncthreads();
  for (int e = t; e < R * R; e += 256) {
    const int a = e / R, b = e % R;
    float s = 0.f;
#pragma unroll 8
    for (int r = 0; r < RB; ++r) s += Zs[r][a] * Zs[r][b];
    Gp[(size_t)blockIdx.x * R * R + e] = s;
  }
}

// The Gram factorisation where no product kernel follows to host it.
template <int R>
__global__ __launch_bounds__(256) void ms_factor_kernel(const float* __restrict__ Gp, int nb,
                                                        float* __restrict__ Mout) {
  __shared__ __attribute__((aligned(16))) float sm[factor_smem<R>()];
  gram_factor<R>(Gp, nb, Mout, sm);
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

// out[o][c] = bf16(W_base[o][c] + (1/k) sum_i sum_j Q_i[o][j] Z_i[c][j]);
// tau (optional) the float32 mean.  A workgroup owns 64 rows x 128 columns,
// wave w the 32 x 64 quarter (w / 2, w % 2).  Per 16-wide block of j, lane
// (n, g) loads Q[row n][4g .. 4g+3] of each 16-row tile (operand A) and
// Z[column n][4g .. 4g+3] of each 16-column tile (operand B); product v
// takes j = 4g + v.  The sums go through LDS so that each thread adds 8
// consecutive columns of a row to W_base with 16-byte accesses.
template <int R>
__global__ __launch_bounds__(256) void ms_merge_kernel(const uint16_t* __restrict__ wb, int d_out,
                                                       int d_in, int k, const float* __restrict__ Q,
                                                       const float* __restrict__ Z,
                                                       uint16_t* __restrict__ out,
                                                       float* __restrict__ tau) {
  constexpr int KB = (R + 15) / 16;
  __shared__ __attribute__((aligned(16))) float C[64][128 + 4];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int o0 = blockIdx.y * 64;
  const int c0 = blockIdx.x * 128;
  const int wr = o0 + 32 * (w >> 1);
  const int wc = c0 + 64 * (w & 1);
  f32x4 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < k; ++i) {
    const float* Qi = Q + (size_t)i * d_out * R;
    const float* Zi = Z + (size_t)i * d_in * R;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int kk = 16 * kb + 4 * g;
      const bool in = kk < R;
      const int kc = in ? kk : 0;
      f32x4 a[2], b[4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f32x4 v =
            *reinterpret_cast<const f32x4*>(Qi + (size_t)min(wr + 16 * u + n, d_out - 1) * R + kc);
        a[u] = in ? v : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 v =
            *reinterpret_cast<const f32x4*>(Zi + (size_t)min(wc + 16 * u + n, d_in - 1) * R + kc);
        b[u] = in ? v : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int ra = 0; ra < 2; ++ra)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) acc[ra][cb] = mfma_f32(a[ra][v], b[cb][v], acc[ra][cb]);
    }
  }
#pragma unroll
  for (int ra = 0; ra < 2; ++ra)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        C[32 * (w >> 1) + 16 * ra + 4 * g + v][64 * (w & 1) + 16 * cb + n] = acc[ra][cb][v];
  __syncthreads();
  const float invk = 1.f / (float)k;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int seg = t + 256 * s;
    const int r = seg >> 4;
    const int cs = (seg & 15) * 8;
    const int o = o0 + r;
    const int c = c0 + cs;
    if (o >= d_out || c >= d_in) continue;
    const size_t base = (size_t)o * d_in + c;
    const u32x4 wv = ld128(wb + base);
    const float4 m0 = *reinterpret_cast<const float4*>(&C[r][cs]);
    const float4 m1 = *reinterpret_cast<const float4*>(&C[r][cs + 4]);
    const float m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    u32x4 res;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float t0 = m[2 * h] * invk;
      const float t1 = m[2 * h + 1] * invk;
      res[h] = (uint32_t)f32_to_bf16_bits(bf16_lo(wv[h]) + t0) |
               ((uint32_t)f32_to_bf16_bits(bf16_hi(wv[h]) + t1) << 16);
      if (tau) {
        tau[base + 2 * h] = t0;
        tau[base + 2 * h + 1] = t1;
      }
    }
    *reinterpret_cast<u32x4*>(out + base) = res;
  }
}

// Workgroups of the epilogue over n rows.
inline int64_t epi_groups(int64_t n) { return (n + kEpiRows - 1) / kEpiRows; }

// Workspace in floats: Y, Z (k planes each), X0, the products' partial
// planes, the Gram partials, the R x R inverse.
struct Layout {
  int64_t y, z, x0, part, gp, m, total;
  Layout(int64_t d_out, int64_t d_in, int k, int64_t R) {
    const int64_t parts = std::max((int64_t)ms_mul_slices(d_out, d_in) * d_out,
                                   (int64_t)ms_tmul_chunks(d_out, d_in) * d_in);
    y = 0;
    z = y + k * d_out * R;
    x0 = z + k * d_in * R;
    part = x0 + d_in * R;
    gp = part + parts * R;
    m = gp + std::max(epi_groups(d_out), epi_groups(d_in)) * R * R;
    total = m + R * R;
  }
};

// One checkpoint's products.  Each epilogue with Gram partials leaves them
// in Gp for `pending` rows; the next product kernel (or a factor kernel)
// turns them into M = U^+, which the epilogue after it applies.
template <int R>
struct Plan {
  int d_out, d_in;
  float *Part, *Gp, *M;
  int64_t pending = 0;  // rows whose Gram partials wait in Gp (0: none)
  hipStream_t s;

  FactorJob job() {
    FactorJob fj{pending ? Gp : nullptr, (int)epi_groups(pending), M};
    pending = 0;
    return fj;
  }
  // A [n][R] = (sum of `parts` partial planes) Min, with Gram partials
  hipError_t epi(const float* P, int parts, int n, const float* Min, float* A, bool gram) {
    hipLaunchKernelGGL(ms_epi_kernel<R>, dim3((unsigned)epi_groups(n)), dim3(256), 0, s, P, parts,
                       n, Min, A, gram ? Gp : nullptr);
    if (gram) pending = n;
    return hipGetLastError();
  }
  hipError_t factor() {
    const FactorJob fj = job();
    if (fj.Gp) hipLaunchKernelGGL(ms_factor_kernel<R>, dim3(1), dim3(256), 0, s, fj.Gp, fj.nb, M);
    return hipGetLastError();
  }
  // Y = (Delta X) M with the pending factorisation (or X's own rows when
  // none is pending), Gram partials of Y
  hipError_t mul(const uint16_t* wf, const uint16_t* wb, const float* X, float* Y) {
    const int ks = ms_mul_slices(d_out, d_in);
    const FactorJob fj = job();
    const int gx = (d_out + 63) / 64 + (fj.Gp ? 1 : 0);
    hipLaunchKernelGGL(ms_mul_kernel<R>, dim3(gx, ks), dim3(256), 0, s, wf, wb, d_out, d_in, ks, X,
                       Part, fj);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : epi(Part, ks, d_out, fj.Gp ? M : nullptr, Y, true);
  }
  // Z = (Delta^T Y) M with the pending factorisation, Gram partials of Z
  // when asked
  hipError_t tmul(const uint16_t* wf, const uint16_t* wb, const float* Y, float* Z, bool gram) {
    const int kt = ms_tmul_chunks(d_out, d_in);
    const FactorJob fj = job();
    const int gx = (d_in + 127) / 128 + (fj.Gp ? 1 : 0);
    hipLaunchKernelGGL(ms_tmul_kernel<R>, dim3(gx, kt), dim3(256), 0, s, wf, wb, d_out, d_in, kt, Y,
                       Part, fj);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : epi(Part, kt, d_in, fj.Gp ? M : nullptr, Z, gram);
  }
};

template <int R>
hipError_t run_monosoup(const uint16_t* const* w_ft, int k, const uint16_t* w_base, int d_out,
                        int d_in, int rank, int q, const float* omega, uint16_t* out, float* tau,
                        char* ws, hipStream_t s) {
  const Layout L(d_out, d_in, k, R);
  float* f = reinterpret_cast<float*>(ws);
  float* const X0 = f + L.x0;
  hipLaunchKernelGGL(ms_pad_kernel, dim3((unsigned)(((size_t)d_in * R + 255) / 256)), dim3(256), 0,
                     s, omega, d_in, rank, R, X0);
  hipError_t e = hipGetLastError();
  for (int i = 0; i < k && e == hipSuccess; ++i) {
    Plan<R> P;
    P.d_out = d_out;
    P.d_in = d_in;
    P.s = s;
    P.Part = f + L.part;
    P.Gp = f + L.gp;
    P.M = f + L.m;
    float* Yi = f + L.y + (size_t)i * d_out * R;
    float* Zi = f + L.z + (size_t)i * d_in * R;
    // Y and Z are stored unscaled; their bases are Y U_Y^+ and Z U_Z^+
    e = P.mul(w_ft[i], w_base, X0, Yi);
    for (int it = 0; it < q && e == hipSuccess; ++it) {
      e = P.tmul(w_ft[i], w_base, Yi, Zi, true);
      if (e == hipSuccess) e = P.mul(w_ft[i], w_base, Zi, Yi);
    }
    // the final basis: a second CholeskyQR pass on the explicit Y U_Y^+,
    // then Z = Delta^T Q and Q itself
    if (e == hipSuccess) e = P.factor();
    if (e == hipSuccess) e = P.epi(Yi, 1, d_out, P.M, Yi, true);
    if (e == hipSuccess) e = P.tmul(w_ft[i], w_base, Yi, Zi, false);
    if (e == hipSuccess) e = P.epi(Yi, 1, d_out, P.M, Yi, false);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ms_merge_kernel<R>, dim3((d_in + 127) / 128, (d_out + 63) / 64), dim3(256),
                     0, s, w_base, d_out, d_in, k, f + L.y, f + L.z, out, tau);
  return hipGetLastError();
}

}  // namespace

int monosoup_width(int rank) { return rank <= 8 ? 8 : (rank <= 16 ? 16 : 32); }

size_t monosoup_workspace_bytes(int64_t d_out, int64_t d_in, int k, int rank) {
  return 4u * (size_t)Layout(d_out, d_in, k, monosoup_width(rank)).total;
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
