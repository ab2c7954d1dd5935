// Prefill-shaped BitDelta linear on gfx950: an LDS-staged bf16 MFMA GEMM
// whose weight tiles are rebuilt on the fly from W_base and the sign bits.
//
// Page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak", section
// "Sunum mimarisi": the effective weight W_eff = W_base + alpha*sign(Delta)
// is formed in fast on-chip memory (here LDS) inside the matmul kernel and
// never written to HBM.
//
// Two kernels, chosen per product by launch_linear_prefill:
//  - prefill_pc_kernel (further below): 512- or 256-token x 128-row tiles
//    with producer waves that stage x and rebuild W_eff beside the MFMA
//    waves; 512-token tiles take the rows that fill whole rounds of the CUs;
//  - prefill_kernel (this comment): 256-token tiles in which every wave both
//    rebuilds and multiplies, 256 or 64 rows wide, for the rest.
//
// prefill_kernel tile: 256 tokens x BN output rows x 64 of d_in per step, 8
// waves as 4 x 2, each owning 64 x (BN/2) outputs in MFMA 32x32x16 tiles
// (float32 accumulators).  Two LDS stages: while the MFMAs read one, the
// other is filled for the next step.  Raw weights are loaded two steps ahead
// into two register sets, so the rebuild of step k+1 (from registers that
// have already arrived) is spread over the four 16-wide MFMA sub-steps of
// step k.
//  * x goes from global memory straight into LDS (buffer loads to LDS, 16
//    bytes per lane, no registers): each wave instruction writes one 8-row
//    block of 1 KB; chunk c of row r sits at position c ^ (r % 8) of its
//    128-byte row and consecutive blocks are 1152 bytes apart, so the MFMA
//    operand reads (32 rows at one chunk) hit distinct banks.
//  * W_base and the sign bytes are buffer loads into registers; each thread
//    rebuilds its 4 x 8 weights as bf16(W_base + alpha*s) and stores them to
//    the weight stage (rows padded to 144 bytes).
// W_eff is rounded to bf16 once per element, the MFMA accumulates in float32
// and y is rounded to bf16.
#include "common.h"
#include "internal.h"

namespace bd {
namespace {

constexpr int BM = 256;
constexpr int kCUs = 256;           // MI355X compute units: one tile per CU per round
constexpr int BK = 64;
constexpr int ABLK = 1152;          // bytes per 8-row block of the x stage (1 KB + 128 B skew)
constexpr int A_STAGE = 32 * ABLK;  // 256 rows
constexpr int LDK = BK + 8;         // weight stage row pitch in bf16 (144 bytes)

// Workgroup barrier without a memory fence.  Callers first wait for their
// own loads and LDS stores, which is what makes the LDS contents visible; the
// memory clobber keeps the compiler from moving memory accesses across the
// barrier.  step_barrier<N> leaves the N most recent vector memory loads in
// flight (s_waitcnt vmcnt(N) lgkmcnt(0)).
template <int N>
__device__ __forceinline__ void step_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("s_barrier" ::: "memory");
}

template <int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void prefill_kernel(
    const uint16_t* __restrict__ x, int M, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ bits8, const float* __restrict__ alpha, int per_row, int d_out,
    int d_in, uint16_t* __restrict__ y, int ldy, int ntm, int ntn, int chunk) {
  constexpr int NT = 64 * WM * WN;   // threads
  constexpr int RS = NT / 8;         // weight rows covered by one pass of 16-byte loads
  constexpr int NB = BN / RS;        // weight pieces per thread per step
  constexpr int AI = 32 / (WM * WN); // 8-row x blocks per wave per step
  constexpr int TMW = BM / WM / 32;  // 32-row MFMA tiles per wave
  constexpr int TNW = BN / WN / 32;  // 32-column MFMA tiles per wave
  static_assert(NB >= 1 && AI >= 1 && TMW >= 1 && TNW >= 1, "tile shape");
  // Separate arrays per stage, so that the compiler sees that reads of one
  // stage do not depend on the LDS loads into the other.
  __shared__ __attribute__((aligned(16))) unsigned char As0[A_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char As1[A_STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs0[BN][LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs1[BN][LDK];

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
  const int lr = T >> 3;  // weight row within an RS-row slab
  const int lc = T & 7;   // 16-byte chunk within the 64-wide step
  const int r8 = lane >> 3;
  const int pos = lane & 7;

  // x: wave wv fills 8-row blocks wv*AI + b; lane (r8, pos) fetches chunk
  // pos ^ r8 of row r8 of the block (rows past M re-read row M-1).  Byte
  // offsets within this tile's rows of x.
  const uint16_t* xbase = x + (size_t)m0 * d_in;
  const int xbytes = min(BM, M - m0) * d_in * 2;
  int xv[AI];
#pragma unroll
  for (int b = 0; b < AI; ++b) {
    const int row = (wv * AI + b) * 8 + r8;
    xv[b] = (min(m0 + row, M - 1) - m0) * d_in * 2 + 16 * (pos ^ r8);
  }
  // W_base and sign bytes of this tile's rows (rows past d_out read zero).
  const int nrows = min(BN, d_out - n0);
  const uint16_t* wbase = w + (size_t)n0 * d_in;
  const int wbytes = nrows * d_in * 2;
  const uint8_t* sbase = bits8 + (size_t)n0 * (d_in >> 3);
  const int sbytes = nrows * (d_in >> 3);
  int vw[NB], vs[NB];
  uint32_t ab[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int r = lr + RS * i;
    vw[i] = (r * d_in + lc * 8) * 2;
    vs[i] = r * (d_in >> 3) + lc;
    ab[i] = __float_as_uint(per_row ? alpha[min(n0 + r, d_out - 1)] : alpha[0]);
  }
  // LDS byte offsets of the x operand for tile i, 16-wide sub-step ks.
  int aoff[TMW][4];
#pragma unroll
  for (int i = 0; i < TMW; ++i) {
    const int r = wm * (BM / WM) + i * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      aoff[i][ks] = (r >> 3) * ABLK + (r & 7) * 128 + ((c ^ (r & 7)) << 4);
    }
  }

  // Two register sets of raw weights: set (k+1)%2 holds step k+1 while step
  // k runs; set k%2 receives step k+2.
  u32x4 rb0[NB], rb1[NB];
  uint32_t rs0[NB], rs1[NB];
  auto xload = [&](int kt, unsigned char* as) {
#pragma unroll
    for (int b = 0; b < AI; ++b)
      lds_bload16(xbase, xbytes, xv[b], kt * BK * 2, as + (wv * AI + b) * ABLK);
  };
  auto wload = [&](int kt, u32x4 (&rb)[NB], uint32_t (&rs)[NB]) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      rb[i] = bload128(wbase, wbytes, vw[i], kt * BK * 2);
      rs[i] = bload8(sbase, sbytes, vs[i], kt * (BK / 8));
    }
  };
  auto wpiece = [&](int i, uint16_t (*bs)[LDK], const u32x4 (&rb)[NB], const uint32_t (&rs)[NB]) {
    *reinterpret_cast<u32x4*>(&bs[lr + RS * i][lc * 8]) = rebuild8(rb[i], rs[i], ab[i]);
  };

  f32x16 acc[TMW][TNW];
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Step kt: stage kt%2 holds x and W_eff of step kt.  Prefetch x of step
  // kt+1 into the other stage and raw W of step kt+2 into rb_load; multiply
  // this stage while rebuilding W_eff of step kt+1 (rb_use) into the other
  // weight stage.  Prefetches are unconditional: past the last step they
  // re-read the last step (in bounds) into buffers nobody reads.
  auto step = [&](int kt, int nk, const unsigned char* as, uint16_t (*bs)[LDK],
                  unsigned char* as_next, uint16_t (*bs_next)[LDK], const u32x4 (&rb_use)[NB],
                  const uint32_t (&rs_use)[NB], u32x4 (&rb_load)[NB], uint32_t (&rs_load)[NB]) {
    xload(min(kt + 1, nk - 1), as_next);
    // x first, then the 2*NB weight loads: the barrier at the end of the
    // step waits for x and leaves the weights (needed one step later) in
    // flight.
    __builtin_amdgcn_sched_barrier(0);
    wload(min(kt + 2, nk - 1), rb_load, rs_load);
    // Keep the prefetches at the top of the step (the scheduler would sink
    // them towards the barrier to save registers).
    __builtin_amdgcn_sched_barrier(0);
    // Operand fragments double-buffered across the 16-wide sub-steps: the
    // reads of sub-step ks+1 are issued before the MFMAs of sub-step ks.
    u32x4 afA[TMW], bfA[TNW], afB[TMW], bfB[TNW];
    auto rd = [&](int ks, u32x4 (&af)[TMW], u32x4 (&bf)[TNW]) {
#pragma unroll
      for (int i = 0; i < TMW; ++i) af[i] = *reinterpret_cast<const u32x4*>(as + aoff[i][ks]);
#pragma unroll
      for (int j = 0; j < TNW; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(
            &bs[wn * (BN / WN) + j * 32 + (lane & 31)][ks * 16 + 8 * (lane >> 5)]);
    };
    auto mm = [&](const u32x4 (&af)[TMW], const u32x4 (&bf)[TNW]) {
#pragma unroll
      for (int i = 0; i < TMW; ++i)
#pragma unroll
        for (int j = 0; j < TNW; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    };
    rd(0, afA, bfA);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ks += 2) {
      rd(ks + 1, afB, bfB);
      mm(afA, bfA);
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (i % 4 == ks) wpiece(i, bs_next, rb_use, rs_use);
      if (ks + 2 < BK / 16) rd(ks + 2, afA, bfA);
      mm(afB, bfB);
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (i % 4 == ks + 1) wpiece(i, bs_next, rb_use, rs_use);
    }
    step_barrier<2 * NB>();
  };

  const int nk = d_in / BK;
  xload(0, As0);
  wload(0, rb0, rs0);
  wload(min(1, nk - 1), rb1, rs1);
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int i = 0; i < NB; ++i) wpiece(i, Bs0, rb0, rs0);
  step_barrier<0>();
  // Steps in unconditional pairs (a conditional second step lets the
  // compiler sink the first step's loads into it), then a last odd step.
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, nk, As0, Bs0, As1, Bs1, rb1, rs1, rb0, rs0);
    step(kt + 1, nk, As1, Bs1, As0, Bs0, rb0, rs0, rb1, rs1);
  }
  if (kt < nk) step(kt, nk, As0, Bs0, As1, Bs1, rb1, rs1, rb0, rs0);

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
        if (m < M && o < d_out) y[(size_t)m * ldy + o] = f32_to_bf16_bits(acc[i][j][v]);
      }
    }
  }
}

// ------------------------------------------------- producer/consumer tiles
// Tile: TBM (512 or 256) tokens x 128 output rows x 64 of d_in per step.
// WM x WN MFMA waves (4 x 2: each (TBM/4) x 64 outputs in MFMA 32x32x16
// tiles) only read the LDS stages and multiply; 4 producer waves follow
// them: they stage x with buffer loads to LDS and rebuild W_eff into the
// next weight stage, so the rebuild's ALU work runs in waves of its own
// beside the MFMA waves instead of inside their instruction streams.  512
// token rows per weight tile halve the rebuild work per MFMA against 256.
// LDS holds two x stages of TBM x 128 bytes and two weight stages of 16 KB
// (160 KB at 512 tokens), rows of 128 bytes with chunk c of row r at
// position c ^ ((r / 2) % 8): the MFMA operand reads (16 consecutive rows at
// one chunk per 256 bytes of banks) are conflict free without padding.  One
// barrier per step for all waves.
constexpr int PC_BM = 512;
constexpr int PC_BN = 128;
constexpr int PC_WSTAGE = PC_BN * 128;
// x of one tile is addressed with 32-bit buffer offsets: 512 rows of d_in.
constexpr int64_t kPcMaxDin = kPrefillMaxTileBytes / (PC_BM * 2) / 64 * 64;
// x larger than this (a quarter of the 256 MB last-level cache) is
// prefetched into L2 two steps ahead.
constexpr int64_t kPcPrefetchXBytes = 64ll << 20;

__device__ __forceinline__ int pc_swz(int r, int c) { return c ^ ((r >> 1) & 7); }

template <bool XPF, int TBM, int WM, int WN>
__global__ __launch_bounds__(64 * (WM * WN + 4), 1) void prefill_pc_kernel(
    const uint16_t* __restrict__ x, int M, const uint16_t* __restrict__ w,
    const uint8_t* __restrict__ bits8, const float* __restrict__ alpha, int per_row, int d_out,
    int d_in, uint16_t* __restrict__ y, int ldy, int ntm, int ntn, int chunk, int xg) {
  constexpr int NMW = WM * WN;          // MFMA waves; 4 producer waves follow
  constexpr int TMW = TBM / WM / 32;    // 32-row MFMA tiles per wave
  constexpr int TNW = PC_BN / WN / 32;  // 32-column MFMA tiles per wave
  constexpr int XSTAGE = TBM * 128;
  static_assert(TMW >= 1 && TNW >= 1, "tile shape");
  static_assert(!XPF || TBM == 512, "x prefetch covers 512 rows");
  constexpr int NB = 4;                 // weight pieces per producer thread per step
  constexpr int AI = TBM / 32;          // 8-row x blocks per producer wave per step
  __shared__ __attribute__((aligned(16))) unsigned char X0[XSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char X1[XSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char W0[PC_WSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char W1[PC_WSTAGE];

  // Workgroups are dealt round-robin to the 8 XCDs.  With xg == 1 each XCD
  // takes a contiguous range of tiles, token tile fastest (as in
  // prefill_kernel); with xg > 1 the token tiles form xg groups and the
  // weight tiles 8 / xg groups (the host checks both divide evenly) and each
  // XCD takes one (token group, weight group) block, so that it fetches a
  // 1/xg share of x into its L2 instead of all of it.
  const int xcd = blockIdx.x & 7;
  const int local = blockIdx.x >> 3;
  int tm, tn;
  if (xg == 1) {
    const int tile = xcd * chunk + local;
    if (tile >= ntm * ntn) return;
    tm = tile % ntm;
    tn = tile / ntm;
  } else {
    const int tmg = ntm / xg;
    tm = (xcd % xg) * tmg + local % tmg;
    tn = (xcd / xg) * (ntn / (8 / xg)) + local / tmg;
  }
  const int m0 = tm * TBM;
  const int n0 = tn * PC_BN;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int nk = d_in / BK;

  if (wv >= NMW) {
    // ------------------------------------------------------------ producers
    const int pw = wv - NMW;
    const int T = threadIdx.x - 64 * NMW;
    const int lr = T >> 3;  // 0..31: weight row within a 32-row pass
    const int lc = T & 7;   // 16-byte chunk within the 64-wide step
    // x rows past M lie beyond the resource and read as zero.  Block b of
    // the tile holds rows 8b..8b+7; lane (r, p) fetches chunk p ^ ((row/2)%8)
    // of row 8b + r, whose swizzle depends on the block's parity only.
    const uint16_t* xbase = x + (size_t)m0 * d_in;
    const int xbytes = min(TBM, M - m0) * d_in * 2;
    int xv[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int row = par * 8 + (lane >> 3);
      xv[par] = row * d_in * 2 + 16 * pc_swz(row, lane & 7);
    }
    // W_base and sign bytes of the tile's rows (rows past d_out read zero);
    // piece i of a thread is row lr + 32 i.
    const int nrows = min(PC_BN, d_out - n0);
    const uint16_t* wbase = w + (size_t)n0 * d_in;
    const int wbytes = nrows * d_in * 2;
    const uint8_t* sbase = bits8 + (size_t)n0 * (d_in >> 3);
    const int sbytes = nrows * (d_in >> 3);
    const int vw0 = (lr * d_in + lc * 8) * 2;
    const int vs0 = lr * (d_in >> 3) + lc;
    const int woff0 = lr * 128 + 16 * pc_swz(lr, lc);  // piece i: + 4096 i, same swizzle
    uint32_t ab[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      ab[i] = __float_as_uint(per_row ? alpha[min(n0 + lr + 32 * i, d_out - 1)] : alpha[0]);
    u32x4 rb0[NB], rb1[NB];
    uint32_t rs0[NB], rs1[NB];
    auto xload = [&](int kt, unsigned char* xs) {
#pragma unroll
      for (int b = 0; b < AI; ++b) {
        const int blk = pw * AI + b;
        lds_bload16(xbase, xbytes, xv[blk & 1], kt * BK * 2 + (blk >> 1) * 16 * d_in * 2,
                    xs + blk * 1024);
      }
    };
    auto wload = [&](int kt, u32x4 (&rb)[NB], uint32_t (&rs)[NB]) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        rb[i] = bload128(wbase, wbytes, vw0, kt * BK * 2 + i * 32 * d_in * 2);
        rs[i] = bload8(sbase, sbytes, vs0, kt * (BK / 8) + i * 32 * (d_in >> 3));
      }
    };
    auto build = [&](unsigned char* ws, const u32x4 (&rb)[NB], const uint32_t (&rs)[NB]) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
        *reinterpret_cast<u32x4*>(ws + woff0 + i * 4096) = rebuild8(rb[i], rs[i], ab[i]);
    };
    // With XPF, one dword of each of the tile's 512 x rows two steps ahead
    // is loaded as well, which brings those 128-byte segments into L2 a step
    // before they are staged (for x too large to stay in the last-level
    // cache).  The loaded values only feed a dummy sum.  The S workgroups of
    // this XCD that stream the same token tile (S a power of two, at most 8)
    // share the work: workgroup i loads rows i, i + S, i + 2S, ... (every
    // line is requested once per L2 instead of S times, and each scattered
    // row costs the address unit several cycles).  Threads with no row of
    // their own read past the end of the buffer, which touches no memory.
    int share = 1, sidx = 0;
    if (xg == 1) {
      if (chunk % ntm == 0) {
        share = chunk / ntm;
        sidx = local / ntm;
      }
    } else {
      share = ntn / (8 / xg);
      sidx = local / (ntm / xg);
    }
    int S = 1;
    while (S < 8 && 2 * S <= share) S *= 2;
    const int npf = TBM / S;  // rows this workgroup prefetches
    uint32_t sink = 0, pf0 = 0, pf1 = 0;
    const int pfv0 = S == 1 ? 2 * T * d_in * 2
                            : (T < npf ? (S * T + sidx % S) * d_in * 2 : xbytes);
    const int pfv1 = S == 1 ? (2 * T + 1) * d_in * 2 : xbytes;
    // Step kt: x of step kt+1 into the free x stage, raw weights of step
    // kt+2 into rb_load, W_eff of step kt+1 (rb_use, loaded a step earlier)
    // into the free weight stage; the barrier waits for x and the LDS
    // stores and leaves the weight loads (and prefetches) in flight.
    // Prefetches past the last step re-read it into buffers nobody reads.
    auto pstep = [&](int kt, unsigned char* xs_next, unsigned char* ws_next,
                     const u32x4 (&rb_use)[NB], const uint32_t (&rs_use)[NB],
                     u32x4 (&rb_load)[NB], uint32_t (&rs_load)[NB]) {
      if constexpr (XPF) sink ^= pf0 ^ pf1;
      xload(min(kt + 1, nk - 1), xs_next);
      __builtin_amdgcn_sched_barrier(0);
      wload(min(kt + 2, nk - 1), rb_load, rs_load);
      if constexpr (XPF) {
        const int so = min(kt + 2, nk - 1) * BK * 2;
        pf0 = bload32(xbase, xbytes, pfv0, so);
        pf1 = bload32(xbase, xbytes, pfv1, so);
      }
      __builtin_amdgcn_sched_barrier(0);
      build(ws_next, rb_use, rs_use);
      step_barrier<2 * NB + (XPF ? 2 : 0)>();
    };
    xload(0, X0);
    wload(0, rb0, rs0);
    wload(min(1, nk - 1), rb1, rs1);
    __builtin_amdgcn_s_waitcnt(0);
    build(W0, rb0, rs0);
    step_barrier<0>();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      pstep(kt, X1, W1, rb1, rs1, rb0, rs0);
      pstep(kt + 1, X0, W0, rb0, rs0, rb1, rs1);
    }
    if (kt < nk) pstep(kt, X1, W1, rb1, rs1, rb0, rs0);
    __builtin_amdgcn_s_waitcnt(0);
    // keeps the prefetch loads alive; d_out is never negative
    if (XPF && (sink ^ pf0 ^ pf1) == 0x9E3779B9u && d_out < 0) y[0] = 0;
    return;
  }

  // ---------------------------------------------------------- MFMA waves
  const int wm = wv % WM;
  const int wn = wv / WM;
  // Operand reads of 16-wide sub-step ks; tile i (j) of the wave lies 32
  // rows (4096 bytes) further on with the same swizzle.
  int aoff[4], boff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c = 2 * ks + (lane >> 5);
    const int ra = wm * (TBM / WM) + (lane & 31);
    aoff[ks] = ra * 128 + 16 * pc_swz(ra, c);
    const int rw = wn * (PC_BN / WN) + (lane & 31);
    boff[ks] = rw * 128 + 16 * pc_swz(rw, c);
  }
  f32x16 acc[TMW][TNW];
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto cstep = [&](const unsigned char* xs, const unsigned char* ws) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 af[TMW], bf[TNW];
#pragma unroll
      for (int i = 0; i < TMW; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(xs + aoff[ks] + i * 4096);
#pragma unroll
      for (int j = 0; j < TNW; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(ws + boff[ks] + j * 4096);
#pragma unroll
      for (int i = 0; i < TMW; ++i)
#pragma unroll
        for (int j = 0; j < TNW; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
    step_barrier<0>();
  };
  step_barrier<0>();  // the producers' first stage
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    cstep(X0, W0);
    cstep(X1, W1);
  }
  if (kt < nk) cstep(X0, W0);

  // MFMA 32x32 output layout as in prefill_kernel.
#pragma unroll
  for (int i = 0; i < TMW; ++i) {
#pragma unroll
    for (int j = 0; j < TNW; ++j) {
      const int o = n0 + wn * (PC_BN / WN) + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * (TBM / WM) + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M && o < d_out) y[(size_t)m * ldy + o] = f32_to_bf16_bits(acc[i][j][v]);
      }
    }
  }
}

// Producer/consumer tiles of TBM tokens x 128 rows over rows [0, d_out) of
// the slab at w (rows of y ldy apart).
template <bool XPF, int TBM, int WM, int WN>
hipError_t launch_pc_cfg(const uint16_t* x, int M, const uint16_t* w, const uint8_t* packed_bytes,
                         const float* alpha, int per_row, int d_out, int d_in, uint16_t* y, int ldy,
                         hipStream_t stream) {
  if (d_in > kPcMaxDin) return hipErrorInvalidValue;
  const int ntm = (M + TBM - 1) / TBM;
  const int ntn = (d_out + PC_BN - 1) / PC_BN;
  const int tiles = ntm * ntn;
  const int chunk = (tiles + 7) / 8;
  // XCD blocks (see the kernel): xg token groups times 8 / xg weight groups
  // where both divide evenly, xg minimising what the 8 L2s fetch between
  // them, 8/xg copies of x plus xg copies of W (ties keep the smaller xg).
  int xg = 1;
  for (int g = 2; g <= 8; g *= 2) {
    if (ntm % g != 0 || ntn % (8 / g) != 0) continue;
    if ((8 / g) * (int64_t)M + g * (int64_t)d_out < (8 / xg) * (int64_t)M + xg * (int64_t)d_out) xg = g;
  }
  hipLaunchKernelGGL((prefill_pc_kernel<XPF, TBM, WM, WN>), dim3(8 * chunk),
                     dim3(64 * (WM * WN + 4)), 0, stream, x, M, w, packed_bytes, alpha, per_row,
                     d_out, d_in, y, ldy, ntm, ntn, chunk, xg);
  return hipGetLastError();
}

hipError_t launch_pc(const uint16_t* x, int M, const uint16_t* w, const uint8_t* packed_bytes,
                     const float* alpha, int per_row, int d_out, int d_in, uint16_t* y, int ldy,
                     hipStream_t stream) {
  // Measured: the L2 prefetch of x pays for the 70B down projection (x of
  // 117 MB, 3% faster) and costs 8-12% where x stays in the last-level cache.
  if ((int64_t)M * d_in * 2 > kPcPrefetchXBytes)
    return launch_pc_cfg<true, PC_BM, 4, 2>(x, M, w, packed_bytes, alpha, per_row, d_out, d_in,
                                            y, ldy, stream);
  return launch_pc_cfg<false, PC_BM, 4, 2>(x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y,
                                           ldy, stream);
}

// Output rows [0, d_out) of the slab starting at w (rows of y are ldy apart).
template <int BN, int WM, int WN>
hipError_t launch_cfg(const uint16_t* x, int M, const uint16_t* w, const uint8_t* packed_bytes,
                      const float* alpha, int per_row, int d_out, int d_in, uint16_t* y, int ldy,
                      hipStream_t stream) {
  // Buffer offsets are 32-bit: one tile's rows of W_base must span < 2 GiB.
  if ((int64_t)BN * d_in * 2 > (int64_t)kPrefillMaxTileBytes) return hipErrorInvalidValue;
  const int ntm = (M + BM - 1) / BM;
  const int ntn = (d_out + BN - 1) / BN;
  const int tiles = ntm * ntn;
  const int chunk = (tiles + 7) / 8;
  hipLaunchKernelGGL((prefill_kernel<BN, WM, WN>), dim3(8 * chunk), dim3(64 * WM * WN), 0, stream,
                     x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y, ldy, ntm, ntn, chunk);
  return hipGetLastError();
}

// 256 tokens x 128 rows: producer/consumer tiles (8 MFMA waves of 64 x 64
// outputs and 4 producers; measured 3-6% faster than the 8-wave kernel's
// 256 x 128 tiles on every shape tried, with identical results).
hipError_t launch_256x128(const uint16_t* x, int M, const uint16_t* w, const uint8_t* packed_bytes,
                          const float* alpha, int per_row, int d_out, int d_in, uint16_t* y,
                          int ldy, hipStream_t stream) {
  if (d_in <= kPcMaxDin)
    return launch_pc_cfg<false, 256, 4, 2>(x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y,
                                           ldy, stream);
  return launch_cfg<128, 4, 2>(x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y, ldy, stream);
}

// Rows [0, d_out) of the slab at w with 256-token tiles (rows of y ldy apart).
hipError_t launch_256(const uint16_t* x, int M, const uint16_t* w, const uint8_t* packed_bytes,
                      const float* alpha, int per_row, int d_out, int d_in, uint16_t* y, int ldy,
                      hipStream_t stream) {
  // 8 waves, two per SIMD; tiles are dealt in rounds over the CUs.
  const long ntm = (M + BM - 1) / BM;
  const long tiles256 = ntm * ((d_out + 255) / 256);
  const long full = tiles256 / kCUs;
  if (full >= 1 && tiles256 % kCUs != 0) {
    // Whole rounds of 256-wide weight tiles, then the remaining rows as
    // 128-wide tiles (twice as many, about half as long), so the last round
    // does not leave part of the chip idle.
    const long n_split = (full * kCUs / ntm) * 256;
    if (n_split > 0 && n_split < d_out) {
      hipError_t e = launch_cfg<256, 4, 2>(x, M, w, packed_bytes, alpha, per_row, (int)n_split,
                                           d_in, y, ldy, stream);
      if (e != hipSuccess) return e;
      return launch_256x128(x, M, w + n_split * d_in, packed_bytes + n_split * (d_in / 8),
                            per_row ? alpha + n_split : alpha, per_row, d_out - (int)n_split,
                            d_in, y + n_split, ldy, stream);
    }
  }
  // Fewer tiles than CUs, or whole rounds: the widest tiles (256, 128, then
  // 64 rows) whose last round leaves at most a quarter of the CUs idle.
  const long rounds256 = (tiles256 + kCUs - 1) / kCUs;
  if (4 * tiles256 >= 3 * kCUs * rounds256)
    return launch_cfg<256, 4, 2>(x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y, ldy,
                                 stream);
  const long tiles128 = ntm * ((d_out + 127) / 128);
  const long rounds128 = (tiles128 + kCUs - 1) / kCUs;
  if (4 * tiles128 >= 3 * kCUs * rounds128)
    return launch_256x128(x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y, ldy, stream);
  return launch_cfg<64, 4, 2>(x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y, ldy, stream);
}

}  // namespace

hipError_t launch_linear_prefill(const uint16_t* x, int M, const uint16_t* w,
                                 const uint8_t* packed_bytes, const float* alpha, int per_row,
                                 int d_out, int d_in, uint16_t* y, hipStream_t stream) {
  // The producer/consumer 512 x 128 tiles take the rows that fill whole
  // rounds over the CUs, when their token padding is at most 10% above that
  // of 256-token tiles; the remaining rows (or the whole product) go to the
  // 256-token tiles.
  const long ntm = (M + BM - 1) / BM;
  const long ntm_pc = (M + PC_BM - 1) / PC_BM;
  if (d_in <= kPcMaxDin && 10 * ntm_pc * PC_BM <= 11 * ntm * BM) {
    const long tiles = ntm_pc * ((d_out + PC_BN - 1) / PC_BN);
    const long full = tiles / kCUs;
    // rows is 0 when the whole rounds hold fewer tiles than one weight tile's
    // column of token tiles (tall x over few rows): then 256-token tiles only.
    const long rows = full < 1 ? 0 : tiles % kCUs == 0 ? d_out : (full * kCUs / ntm_pc) * PC_BN;
    if (rows > 0) {
      if (rows >= d_out)
        return launch_pc(x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y, d_out, stream);
      hipError_t e =
          launch_pc(x, M, w, packed_bytes, alpha, per_row, (int)rows, d_in, y, d_out, stream);
      if (e != hipSuccess) return e;
      return launch_256(x, M, w + rows * d_in, packed_bytes + rows * (d_in / 8),
                        per_row ? alpha + rows : alpha, per_row, d_out - (int)rows, d_in,
                        y + rows, d_out, stream);
    }
  }
  return launch_256(x, M, w, packed_bytes, alpha, per_row, d_out, d_in, y, d_out, stream);
}

}  // namespace bd
