// C ABI of libbitdelta: argument checks, device check and kernel dispatch.
// Every check runs on the host before anything is enqueued; see
// include/bitdelta.h for the contract of each entry point.
#include <atomic>
#include <cstring>
#include <mutex>

#include "bitdelta.h"
#include "common.h"
#include "internal.h"
#include "probe.h"
#include "scale_round.h"

#define BD_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kInt32Max = 2147483647;
constexpr int64_t kMaxElems = int64_t(1) << 40;
// The MonoSoup merge kernel's grid takes 64 rows per workgroup in its y
// dimension (at most 65535 workgroups).
constexpr int64_t kMonosoupMaxRows = 65535 * 64;
// The product Delta X addresses a workgroup's 64 rows of each matrix with
// 32-bit buffer offsets: 64 d_in bf16 values must stay below 2 GiB.
constexpr int64_t kMonosoupMaxCols = (int64_t(1) << 24) - 64;

// Row lengths up to 2^30 keep every per-row element and chunk index of the
// kernels (a row's chunks of 512 elements, rounded up) inside a 32-bit int.
constexpr int64_t kMaxDin = int64_t(1) << 30;

bool shape_ok(int64_t d_out, int64_t d_in) {
  return d_out >= 1 && d_in >= 64 && d_in % 64 == 0 && d_out <= kInt32Max && d_in <= kMaxDin &&
         d_out * d_in < kMaxElems;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// 0 unknown, 1 gfx950, 2 other.  Cached per device index.
std::atomic<int> g_arch_state[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BITDELTA_ERR_HIP;
  if (dev < 0 || dev >= 64) return BITDELTA_ERR_DEVICE;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BITDELTA_ERR_HIP;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? BITDELTA_OK : BITDELTA_ERR_DEVICE;
}

int status_of(hipError_t e) { return e == hipSuccess ? BITDELTA_OK : BITDELTA_ERR_HIP; }

}  // namespace

BD_EXPORT const char* bitdelta_status_string(int status) {
  switch (status) {
    case BITDELTA_OK: return "ok";
    case BITDELTA_ERR_NULL: return "a required pointer is NULL";
    case BITDELTA_ERR_SHAPE:
      return "shape out of range (need M >= 1, d_out >= 1, d_in >= 64, d_in % 64 == 0, "
             "each below 2^31, d_out*d_in below 2^40)";
    case BITDELTA_ERR_ALIGN: return "a buffer is not 16-byte aligned";
    case BITDELTA_ERR_MODE: return "alpha_mode must be 0 (per matrix) or 1 (per row)";
    case BITDELTA_ERR_VARIANTS: return "n_variants must be in [1, 64]";
    case BITDELTA_ERR_WORKSPACE: return "workspace missing or too small";
    case BITDELTA_ERR_HIP: return "HIP runtime error";
    case BITDELTA_ERR_DEVICE: return "current device is not a gfx950 GPU";
    case BITDELTA_ERR_OVERLAP: return "an output buffer overlaps an input buffer";
    case BITDELTA_ERR_CACHE:
      return "delta cache: parameter or variant out of range, or call out of order";
    default: return "unknown status";
  }
}

BD_EXPORT uint32_t bitdelta_ratio_to_f32_bits(uint64_t s_hi, uint64_t s_lo, uint64_t n) {
  return bd::ratio_to_f32_bits(s_hi, s_lo, n);
}

BD_EXPORT size_t bitdelta_compress_workspace_size(int64_t d_out, int64_t d_in, int alpha_mode) {
  if (!shape_ok(d_out, d_in)) return 0;
  if (alpha_mode == BITDELTA_ALPHA_PER_MATRIX) return (size_t)d_out * 16u;
  return 0;
}

BD_EXPORT int bitdelta_compress(const uint16_t* w_ft, const uint16_t* w_base, int64_t d_out,
                                int64_t d_in, int alpha_mode, uint64_t* packed, float* alpha,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!w_ft || !w_base || !packed || !alpha) return BITDELTA_ERR_NULL;
  if (!shape_ok(d_out, d_in)) return BITDELTA_ERR_SHAPE;
  if (alpha_mode != BITDELTA_ALPHA_PER_MATRIX && alpha_mode != BITDELTA_ALPHA_PER_ROW)
    return BITDELTA_ERR_MODE;
  if (!aligned16(w_ft) || !aligned16(w_base) || !aligned16(packed) || !aligned16(alpha))
    return BITDELTA_ERR_ALIGN;
  const size_t need = bitdelta_compress_workspace_size(d_out, d_in, alpha_mode);
  if (need > 0 && (!workspace || workspace_bytes < need)) return BITDELTA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return BITDELTA_ERR_ALIGN;
  const size_t wbytes = (size_t)d_out * (size_t)d_in * 2u;
  const size_t pbytes = wbytes / 16u;
  const size_t abytes = alpha_mode == BITDELTA_ALPHA_PER_ROW ? (size_t)d_out * 4u : 4u;
  if (overlap(packed, pbytes, w_ft, wbytes) || overlap(packed, pbytes, w_base, wbytes) ||
      overlap(alpha, abytes, w_ft, wbytes) || overlap(alpha, abytes, w_base, wbytes) ||
      overlap(alpha, abytes, packed, pbytes) ||
      (need > 0 && (overlap(workspace, need, w_ft, wbytes) ||
                    overlap(workspace, need, w_base, wbytes) ||
                    overlap(workspace, need, packed, pbytes) ||
                    overlap(workspace, need, alpha, abytes))))
    return BITDELTA_ERR_OVERLAP;
  const int dev = check_device();
  if (dev != BITDELTA_OK) return dev;
  return status_of(bd::launch_compress(w_ft, w_base, (int)d_out, (int)d_in,
                                       alpha_mode == BITDELTA_ALPHA_PER_ROW, packed, alpha,
                                       static_cast<uint64_t*>(workspace),
                                       static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ no-alloc
// Scratch of bitdelta_compress_noalloc: the per-row integer partial sums of a
// per-matrix scale (16 bytes per row), in a file-scope device array instead
// of a caller workspace.  Each GPU holds its own copy for the life of the
// process.  Host code never uses the array's name as an address: the device
// address is looked up once per device, with that device current, and kept.
constexpr int64_t kNoAllocMaxRows = 262144;  // 4 MiB of scratch
static __device__ __align__(256) uint64_t scratch[2 * kNoAllocMaxRows];

namespace {
void* g_scratch_ptr[64];
hipError_t g_scratch_err[64];
std::once_flag g_scratch_once[64];

// Device address of this device's scratch (nullptr on failure, with *err set).
void* scratch_on_current_device(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}
}  // namespace

BD_EXPORT int bitdelta_compress_noalloc(const uint16_t* w_ft, const uint16_t* w_base,
                                        int64_t d_out, int64_t d_in, int alpha_mode,
                                        uint64_t* packed, float* alpha, void* stream) {
  if (!w_ft || !w_base || !packed || !alpha) return BITDELTA_ERR_NULL;
  if (!shape_ok(d_out, d_in)) return BITDELTA_ERR_SHAPE;
  if (alpha_mode != BITDELTA_ALPHA_PER_MATRIX && alpha_mode != BITDELTA_ALPHA_PER_ROW)
    return BITDELTA_ERR_MODE;
  if (alpha_mode == BITDELTA_ALPHA_PER_MATRIX && d_out > kNoAllocMaxRows)
    return BITDELTA_ERR_WORKSPACE;
  if (!aligned16(w_ft) || !aligned16(w_base) || !aligned16(packed) || !aligned16(alpha))
    return BITDELTA_ERR_ALIGN;
  const size_t wbytes = (size_t)d_out * (size_t)d_in * 2u;
  const size_t pbytes = wbytes / 16u;
  const size_t abytes = alpha_mode == BITDELTA_ALPHA_PER_ROW ? (size_t)d_out * 4u : 4u;
  if (overlap(packed, pbytes, w_ft, wbytes) || overlap(packed, pbytes, w_base, wbytes) ||
      overlap(alpha, abytes, w_ft, wbytes) || overlap(alpha, abytes, w_base, wbytes) ||
      overlap(alpha, abytes, packed, pbytes))
    return BITDELTA_ERR_OVERLAP;
  const int dev = check_device();
  if (dev != BITDELTA_OK) return dev;
  uint64_t* partial = nullptr;
  if (alpha_mode == BITDELTA_ALPHA_PER_MATRIX) {
    hipError_t e = hipSuccess;
    partial = static_cast<uint64_t*>(scratch_on_current_device(&e));
    if (e != hipSuccess || !partial) return BITDELTA_ERR_HIP;
  }
  // The row pass writes both limbs of every row 0..d_out-1 before the
  // finalize reads them, so nothing left by an earlier call is ever read.
  return status_of(bd::launch_compress(w_ft, w_base, (int)d_out, (int)d_in,
                                       alpha_mode == BITDELTA_ALPHA_PER_ROW, packed, alpha,
                                       partial, static_cast<hipStream_t>(stream)));
}

BD_EXPORT int bitdelta_linear(const uint16_t* x, int64_t M, const uint16_t* w_base,
                              const uint64_t* packed, const float* alpha, int alpha_mode,
                              int64_t d_out, int64_t d_in, uint16_t* y, void* stream) {
  if (!x || !w_base || !packed || !alpha || !y) return BITDELTA_ERR_NULL;
  if (!shape_ok(d_out, d_in) || M < 1 || M > kInt32Max || M * d_in >= kMaxElems ||
      M * d_out >= kMaxElems ||
      d_in > (M > bd::kMaxSkinnyTokens ? bd::kPrefillMaxDin : bd::kSkinnyMaxDin))
    return BITDELTA_ERR_SHAPE;
  if (alpha_mode != BITDELTA_ALPHA_PER_MATRIX && alpha_mode != BITDELTA_ALPHA_PER_ROW)
    return BITDELTA_ERR_MODE;
  if (!aligned16(x) || !aligned16(w_base) || !aligned16(packed) || !aligned16(y))
    return BITDELTA_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(alpha) & 3u) return BITDELTA_ERR_ALIGN;
  const size_t ybytes = (size_t)M * (size_t)d_out * 2u;
  const size_t wbytes = (size_t)d_out * (size_t)d_in * 2u;
  const size_t abytes = alpha_mode == BITDELTA_ALPHA_PER_ROW ? (size_t)d_out * 4u : 4u;
  if (overlap(y, ybytes, x, (size_t)M * (size_t)d_in * 2u) || overlap(y, ybytes, w_base, wbytes) ||
      overlap(y, ybytes, packed, wbytes / 16u) || overlap(y, ybytes, alpha, abytes))
    return BITDELTA_ERR_OVERLAP;
  const int dev = check_device();
  if (dev != BITDELTA_OK) return dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M <= bd::kMaxSkinnyTokens) {
    bd::SkinnyArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = x;
    a.ids = nullptr;
    a.w = w_base;
    a.y = y;
    a.M = (int)M;
    a.d_out = (int)d_out;
    a.d_in = (int)d_in;
    a.per_row = alpha_mode == BITDELTA_ALPHA_PER_ROW;
    a.n_variants = 1;
    a.packed[0] = reinterpret_cast<const uint32_t*>(packed);
    a.alpha[0] = alpha;
    return status_of(bd::launch_linear_skinny(a, s));
  }
  return status_of(bd::launch_linear_prefill(
      x, (int)M, w_base, reinterpret_cast<const uint8_t*>(packed), alpha,
      alpha_mode == BITDELTA_ALPHA_PER_ROW, (int)d_out, (int)d_in, y, s));
}

BD_EXPORT int bitdelta_linear_multi(const uint16_t* x, int64_t M, const int32_t* variant_ids,
                                    const uint16_t* w_base, int32_t n_variants,
                                    const uint64_t* const* packed, const float* const* alpha,
                                    int alpha_mode, int64_t d_out, int64_t d_in, uint16_t* y,
                                    void* stream) {
  if (!x || !variant_ids || !w_base || !packed || !alpha || !y) return BITDELTA_ERR_NULL;
  if (!shape_ok(d_out, d_in) || M < 1 || M > kInt32Max || M * d_in >= kMaxElems ||
      M * d_out >= kMaxElems || d_in > bd::kSkinnyMaxDin)
    return BITDELTA_ERR_SHAPE;
  if (alpha_mode != BITDELTA_ALPHA_PER_MATRIX && alpha_mode != BITDELTA_ALPHA_PER_ROW)
    return BITDELTA_ERR_MODE;
  if (n_variants < 1 || n_variants > BITDELTA_MAX_VARIANTS) return BITDELTA_ERR_VARIANTS;
  for (int v = 0; v < n_variants; ++v)
    if (!packed[v] || !alpha[v]) return BITDELTA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_base) || !aligned16(y) ||
      (reinterpret_cast<uintptr_t>(variant_ids) & 3u))
    return BITDELTA_ERR_ALIGN;
  for (int v = 0; v < n_variants; ++v)
    if (!aligned16(packed[v]) || (reinterpret_cast<uintptr_t>(alpha[v]) & 3u))
      return BITDELTA_ERR_ALIGN;
  const size_t ybytes = (size_t)M * (size_t)d_out * 2u;
  const size_t wbytes = (size_t)d_out * (size_t)d_in * 2u;
  const size_t abytes = alpha_mode == BITDELTA_ALPHA_PER_ROW ? (size_t)d_out * 4u : 4u;
  if (overlap(y, ybytes, x, (size_t)M * (size_t)d_in * 2u) || overlap(y, ybytes, w_base, wbytes) ||
      overlap(y, ybytes, variant_ids, (size_t)M * 4u))
    return BITDELTA_ERR_OVERLAP;
  for (int v = 0; v < n_variants; ++v)
    if (overlap(y, ybytes, packed[v], wbytes / 16u) || overlap(y, ybytes, alpha[v], abytes))
      return BITDELTA_ERR_OVERLAP;
  const int dev = check_device();
  if (dev != BITDELTA_OK) return dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bd::SkinnyArgs a;
  std::memset(&a, 0, sizeof(a));
  a.w = w_base;
  a.d_out = (int)d_out;
  a.d_in = (int)d_in;
  a.per_row = alpha_mode == BITDELTA_ALPHA_PER_ROW;
  a.n_variants = n_variants;
  for (int v = 0; v < n_variants; ++v) {
    a.packed[v] = reinterpret_cast<const uint32_t*>(packed[v]);
    a.alpha[v] = alpha[v];
  }
  for (int64_t m0 = 0; m0 < M; m0 += bd::kMaxSkinnyTokens) {
    const int mc = (int)((M - m0) < bd::kMaxSkinnyTokens ? (M - m0) : bd::kMaxSkinnyTokens);
    a.x = x + m0 * d_in;
    a.ids = variant_ids + m0;
    a.y = y + m0 * d_out;
    a.M = mc;
    const int st = status_of(bd::launch_linear_multi(a, s));
    if (st != BITDELTA_OK) return st;
  }
  return BITDELTA_OK;
}

BD_EXPORT int bitdelta_reconstruct(const uint16_t* w_base, const uint64_t* packed,
                                   const float* alpha, int alpha_mode, int64_t d_out,
                                   int64_t d_in, uint16_t* w_eff, void* stream) {
  if (!w_base || !packed || !alpha || !w_eff) return BITDELTA_ERR_NULL;
  if (!shape_ok(d_out, d_in)) return BITDELTA_ERR_SHAPE;
  if (alpha_mode != BITDELTA_ALPHA_PER_MATRIX && alpha_mode != BITDELTA_ALPHA_PER_ROW)
    return BITDELTA_ERR_MODE;
  if (!aligned16(w_base) || !aligned16(packed) || !aligned16(w_eff)) return BITDELTA_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(alpha) & 3u) return BITDELTA_ERR_ALIGN;
  const size_t wbytes = (size_t)d_out * (size_t)d_in * 2u;
  const size_t abytes = alpha_mode == BITDELTA_ALPHA_PER_ROW ? (size_t)d_out * 4u : 4u;
  if (overlap(w_eff, wbytes, w_base, wbytes) || overlap(w_eff, wbytes, packed, wbytes / 16u) ||
      overlap(w_eff, wbytes, alpha, abytes))
    return BITDELTA_ERR_OVERLAP;
  const int dev = check_device();
  if (dev != BITDELTA_OK) return dev;
  return status_of(bd::launch_reconstruct(w_base, reinterpret_cast<const uint8_t*>(packed), alpha,
                                          alpha_mode == BITDELTA_ALPHA_PER_ROW, (int)d_out,
                                          (int)d_in, w_eff, static_cast<hipStream_t>(stream)));
}

BD_EXPORT size_t bitdelta_monosoup_workspace_size(int64_t d_out, int64_t d_in, int32_t k,
                                                  int32_t rank) {
  if (!shape_ok(d_out, d_in) || k < 1 || k > BITDELTA_MONOSOUP_MAX_CHECKPOINTS || rank < 1 ||
      rank > BITDELTA_MONOSOUP_MAX_RANK || rank > d_out || rank > d_in ||
      d_out > kMonosoupMaxRows || d_in > kMonosoupMaxCols)
    return 0;
  return bd::monosoup_workspace_bytes(d_out, d_in, k, rank);
}

BD_EXPORT int bitdelta_monosoup_merge(const uint16_t* const* w_ft, int32_t k,
                                      const uint16_t* w_base, int64_t d_out, int64_t d_in,
                                      int32_t rank, int32_t power_iters, const float* omega,
                                      uint16_t* w_merged, float* tau_mean, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (!w_ft || !w_base || !omega || !w_merged || !workspace) return BITDELTA_ERR_NULL;
  if (!shape_ok(d_out, d_in) || k < 1 || k > BITDELTA_MONOSOUP_MAX_CHECKPOINTS || rank < 1 ||
      rank > BITDELTA_MONOSOUP_MAX_RANK || rank > d_out || rank > d_in || power_iters < 0 ||
      power_iters > BITDELTA_MONOSOUP_MAX_POWER_ITERS || d_out * d_in >= kMaxElems / 4 ||
      d_out > kMonosoupMaxRows || d_in > kMonosoupMaxCols)
    return BITDELTA_ERR_SHAPE;
  for (int i = 0; i < k; ++i)
    if (!w_ft[i]) return BITDELTA_ERR_NULL;
  for (int i = 0; i < k; ++i)
    if (!aligned16(w_ft[i])) return BITDELTA_ERR_ALIGN;
  if (!aligned16(w_base) || !aligned16(w_merged) || !aligned16(workspace) ||
      (tau_mean && !aligned16(tau_mean)) || (reinterpret_cast<uintptr_t>(omega) & 3u))
    return BITDELTA_ERR_ALIGN;
  const size_t need = bd::monosoup_workspace_bytes(d_out, d_in, k, rank);
  if (workspace_bytes < need) return BITDELTA_ERR_WORKSPACE;
  const size_t wbytes = (size_t)d_out * (size_t)d_in * 2u;
  const size_t tbytes = wbytes * 2u;
  const size_t obytes = (size_t)d_in * (size_t)rank * 4u;
  const void* outs[3] = {w_merged, tau_mean, workspace};
  const size_t outn[3] = {wbytes, tbytes, need};
  for (int a = 0; a < 3; ++a) {
    if (!outs[a]) continue;
    if (overlap(outs[a], outn[a], w_base, wbytes) || overlap(outs[a], outn[a], omega, obytes))
      return BITDELTA_ERR_OVERLAP;
    for (int i = 0; i < k; ++i)
      if (overlap(outs[a], outn[a], w_ft[i], wbytes)) return BITDELTA_ERR_OVERLAP;
    for (int b = a + 1; b < 3; ++b)
      if (outs[b] && overlap(outs[a], outn[a], outs[b], outn[b])) return BITDELTA_ERR_OVERLAP;
  }
  const int dev = check_device();
  if (dev != BITDELTA_OK) return dev;
  return status_of(bd::launch_monosoup(w_ft, k, w_base, (int)d_out, (int)d_in, rank, power_iters,
                                       omega, w_merged, tau_mean, workspace,
                                       static_cast<hipStream_t>(stream)));
}

BD_EXPORT int bitdelta_probe_stream_read(const void* src, size_t bytes, int32_t workgroups,
                                         uint32_t* sink, void* stream) {
  if (!src || !sink) return BITDELTA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > (1 << 20))
    return BITDELTA_ERR_SHAPE;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return BITDELTA_ERR_ALIGN;
  if (overlap(sink, 1024, src, bytes)) return BITDELTA_ERR_OVERLAP;
  const int dev = check_device();
  if (dev != BITDELTA_OK) return dev;
  return status_of(bd::launch_probe_read(src, bytes, workgroups, sink,
                                         static_cast<hipStream_t>(stream)));
}

BD_EXPORT int bitdelta_probe_decode_loads(const void* w, const void* signs, const void* x,
                                          int32_t mode, uint32_t* sink, void* stream) {
  if (!w || !signs || !x || !sink) return BITDELTA_ERR_NULL;
  if (mode < 0 || mode > 5) return BITDELTA_ERR_MODE;
  if (!aligned16(w) || !aligned16(x) || (reinterpret_cast<uintptr_t>(signs) & 3u) ||
      (reinterpret_cast<uintptr_t>(sink) & 3u))
    return BITDELTA_ERR_ALIGN;
  if (overlap(sink, 1024, w, size_t(4096) * 8192) || overlap(sink, 1024, signs, size_t(1) << 21) ||
      overlap(sink, 1024, x, 8192))
    return BITDELTA_ERR_OVERLAP;
  const int dev = check_device();
  if (dev != BITDELTA_OK) return dev;
  return status_of(bd::launch_probe_decode_loads(w, signs, x, mode, sink,
                                                 static_cast<hipStream_t>(stream)));
}

BD_EXPORT int bitdelta_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* sink,
                                       void* stream) {
  if (!sink) return BITDELTA_ERR_NULL;
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24))
    return BITDELTA_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(sink) & 3u) return BITDELTA_ERR_ALIGN;
  const int dev = check_device();
  if (dev != BITDELTA_OK) return dev;
  return status_of(bd::launch_probe_mfma(workgroups, iters, sink,
                                         static_cast<hipStream_t>(stream)));
}
