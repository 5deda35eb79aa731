// Host side of the C ABI: argument checks, error text, dispatch.
#include <cmath>
#include <cstdarg>
#include <cstring>
#include <mutex>

#include "had_internal.h"

namespace had {

static thread_local char g_last_error[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

had_status failf(had_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

had_status check_shape(const had_shape& s, int64_t max_seq) {
  if (s.batch <= 0 || s.heads <= 0 || s.seq <= 0 || s.dim <= 0)
    return fail(HAD_ERR_INVALID_ARG, "shape fields must all be positive");
  if (s.dim > HAD_MAX_DIM) return fail(HAD_ERR_UNSUPPORTED, "dim above HAD_MAX_DIM (256)");
  if (s.seq > max_seq) return failf(HAD_ERR_UNSUPPORTED, "seq above the limit (%lld)", static_cast<long long>(max_seq));
  const double total = static_cast<double>(s.batch) * s.heads * s.seq * s.dim;
  if (total > 9.0e15) return fail(HAD_ERR_UNSUPPORTED, "tensor too large");
  if (static_cast<double>(s.batch) * s.heads > 2.0e9)
    return fail(HAD_ERR_UNSUPPORTED, "batch*heads too large");
  return HAD_OK;
}

static had_status check_bits(const uint32_t* qbits, const uint32_t* kbits, const char* fn) {
  if (qbits == nullptr || kbits == nullptr) {
    set_error("%s: null qbits or kbits", fn);
    return HAD_ERR_INVALID_ARG;
  }
  if (!aligned(qbits, 4) || !aligned(kbits, 4)) {
    set_error("%s: qbits and kbits must be 4-byte aligned", fn);
    return HAD_ERR_INVALID_ARG;
  }
  return HAD_OK;
}

}  // namespace had

using namespace had;

extern "C" int64_t had_words_per_row(int64_t dim) { return dim > 0 ? words_per_row(dim) : 0; }

extern "C" const char* had_status_string(had_status st) {
  // A C caller may pass any int: read the argument's bytes as one instead of
  // loading a possibly out-of-range enum value.
  int v;
  static_assert(sizeof(v) == sizeof(st), "had_status is int-sized");
  std::memcpy(&v, &st, sizeof(v));
  switch (v) {
    case HAD_OK: return "HAD_OK";
    case HAD_ERR_INVALID_ARG: return "HAD_ERR_INVALID_ARG";
    case HAD_ERR_UNSUPPORTED: return "HAD_ERR_UNSUPPORTED";
    case HAD_ERR_HIP: return "HAD_ERR_HIP";
  }
  return "HAD_ERR_UNKNOWN";
}

extern "C" const char* had_last_error(void) { return g_last_error; }

// Checks of had_attention's arguments; fills the launch arguments.
static had_status attend_args(const uint32_t* qbits, const uint32_t* kbits, const void* v,
                              int v_dtype, const had_shape& s, int64_t topn, float scale,
                              int causal, float* out, const char* fn, AttnArgs& a) {
  had_status st;
  if ((st = check_bits(qbits, kbits, fn)) != HAD_OK) return st;
  if (v == nullptr || out == nullptr) return failf(HAD_ERR_INVALID_ARG, "%s: null v or out", fn);
  if (!aligned(v, 16) || !aligned(out, 16))
    return failf(HAD_ERR_INVALID_ARG, "%s: v and out must be 16-byte aligned", fn);
  if (!valid_dtype(v_dtype)) return failf(HAD_ERR_INVALID_ARG, "%s: unknown v_dtype", fn);
  if (topn < 1) return failf(HAD_ERR_INVALID_ARG, "%s: topn must be >= 1", fn);
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return failf(HAD_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  if (causal != 0 && causal != 1) return failf(HAD_ERR_INVALID_ARG, "%s: causal must be 0 or 1", fn);
  a = AttnArgs{};
  a.qbits = qbits;
  a.kbits = kbits;
  a.v = v;
  a.v_dtype = static_cast<had_dtype>(v_dtype);
  a.bh_total = s.batch * s.heads;
  a.bh_begin = 0;
  a.bh_count = a.bh_total;
  a.n = static_cast<int>(s.seq);
  a.d = static_cast<int>(s.dim);
  a.topn = static_cast<int>(topn > s.seq ? s.seq : topn);
  a.scale = scale;
  a.causal = causal;
  a.out = out;
  return HAD_OK;
}

extern "C" had_status had_attention(const uint32_t* qbits, const uint32_t* kbits, const void* v,
                                    had_dtype v_dtype, had_shape s, int64_t topn, float scale,
                                    int causal, float* out, void* stream) {
  clear_error();
  had_status st = check_shape(s);
  if (st != HAD_OK) return st;
  AttnArgs a;
  if ((st = attend_args(qbits, kbits, v, enum_bits(v_dtype), s, topn, scale, causal, out, "had_attention", a)) !=
      HAD_OK)
    return st;
  return launch_attention_family(AttnMode::Attend, a, static_cast<hipStream_t>(stream));
}

extern "C" size_t had_forward_workspace_bytes(had_shape s) {
  if (check_shape(s) != HAD_OK) return 0;
#if HAD_FUSED_QPACK
  // the K partials (after an unused Q slot), then one pair per attend wave
  return 2 * had_pack_workspace_bytes(s) + 2 * sizeof(double) * static_cast<size_t>(attend_wave_count(s));
#else
  return 2 * had_pack_workspace_bytes(s);
#endif
}

namespace had {
namespace {

// The two launches of the forward call; ws holds 2 * pack_partials(s) partial
// pairs per tensor that asks for sigma (checked by the caller).
had_status forward_launch(const float* q, const float* k, const void* v, int v_dtype,
                          const had_shape& s, int64_t topn, float scale, int causal,
                          uint32_t* qbits, uint32_t* kbits, float* out, float* sigma_q,
                          float* sigma_k, double* ws, uint32_t* dev_status, hipStream_t hs,
                          const char* who) {
  had_status st;
  if ((st = check_pack_args(q, qbits, sigma_q, who)) != HAD_OK) return st;
  if ((st = check_pack_args(k, kbits, sigma_k, who)) != HAD_OK) return st;
  if (dev_status != nullptr && !aligned(dev_status, 4))
    return failf(HAD_ERR_INVALID_ARG, "%s: dev_status must be 4-byte aligned", who);
  AttnArgs a;
  if ((st = attend_args(qbits, kbits, v, v_dtype, s, topn, scale, causal, out, who, a)) != HAD_OK)
    return st;
  double* part[2] = {nullptr, nullptr};
  if (sigma_q != nullptr) part[0] = ws;
  if (sigma_k != nullptr) part[1] = ws + 2 * pack_partials(s);
  const double count = static_cast<double>(s.batch * s.heads * s.seq) * static_cast<double>(s.dim);
#if HAD_FUSED_QPACK
  // measurement build: K is packed by its own launch, Q inside the attend
  // launch (one sigma partial pair per wave), then sigma_Q from those pairs
  const PackJob kjob{k, kbits, part[1]};
  if ((st = launch_pack(&kjob, 1, s, dev_status, hs)) != HAD_OK) return st;
  if (!aligned(q, 4)) return failf(HAD_ERR_INVALID_ARG, "%s: q must be 4-byte aligned", who);
  double* qpart = sigma_q != nullptr ? ws + 4 * pack_partials(s) : nullptr;
  a.qf = q;
  a.qf_vec = aligned(q, 16) && s.dim == 32 * words_per_row(s.dim) ? 1 : 0;
  a.qbits_out = qbits;
  a.qpartials = qpart;
  a.dev_status = dev_status;
  a.sigma_partials[1] = reinterpret_cast<const double2*>(part[1]);
  a.sigma_out[1] = sigma_k;
  a.sigma_nparts = pack_partials(s);
  a.sigma_count = count;
  if ((st = launch_attention_family(AttnMode::Attend, a, hs)) != HAD_OK) return st;
  if (sigma_q == nullptr) return HAD_OK;
  return launch_sigma_finalize_n(qpart, attend_wave_count(s), count, sigma_q, hs);
#else
  const PackJob jobs[2] = {{q, qbits, part[0]}, {k, kbits, part[1]}};
  if ((st = launch_pack(jobs, 2, s, dev_status, hs)) != HAD_OK) return st;
  a.sigma_partials[0] = reinterpret_cast<const double2*>(part[0]);
  a.sigma_partials[1] = reinterpret_cast<const double2*>(part[1]);
  a.sigma_out[0] = sigma_q;
  a.sigma_out[1] = sigma_k;
  a.sigma_nparts = pack_partials(s);
  a.sigma_count = count;
  return launch_attention_family(AttnMode::Attend, a, hs);
#endif
}

}  // namespace
}  // namespace had

extern "C" had_status had_forward(const float* q, const float* k, const void* v, had_dtype v_dtype,
                                  had_shape s, int64_t topn, float scale, int causal,
                                  uint32_t* qbits, uint32_t* kbits, float* out, float* sigma_q,
                                  float* sigma_k, void* workspace, size_t workspace_bytes,
                                  uint32_t* dev_status, void* stream) {
  clear_error();
  had_status st = check_shape(s);
  if (st != HAD_OK) return st;
  if (sigma_q != nullptr || sigma_k != nullptr) {
    if (workspace == nullptr || !aligned(workspace, 16))
      return fail(HAD_ERR_INVALID_ARG, "had_forward: sigma requested but workspace is null or unaligned");
    if (workspace_bytes < had_forward_workspace_bytes(s))
      return fail(HAD_ERR_INVALID_ARG, "had_forward: workspace smaller than had_forward_workspace_bytes()");
  }
  return forward_launch(q, k, v, enum_bits(v_dtype), s, topn, scale, causal, qbits, kbits, out, sigma_q,
                        sigma_k, static_cast<double*>(workspace), dev_status, static_cast<hipStream_t>(stream),
                        "had_forward");
}

// ---- had_forward_noalloc: the forward call with its sigma partials in a
// file-scope device array instead of a caller workspace.  Every GPU the
// library runs on holds its own copy of the array until the process ends;
// its address on each device is looked up once (hipGetSymbolAddress, with
// that device current) and kept.  The array's name is only a host-side stand-in for
// the symbol: host code passes the looked-up address, never the name.
namespace had {
namespace {

constexpr size_t kScratchBytes = HAD_FORWARD_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes >= 2 * kPackMaxBlocks * 2 * sizeof(double),
              "scratch must hold the sigma partials of the largest pack grid");
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // guarded by g_scratch_mu; null until looked up

// Device address of this device's scratch array for work on stream st.
had_status scratch_address(hipStream_t st, void** ptr) {
  int dev = -1;
  hipError_t e = st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return failf(HAD_ERR_HIP, "had_forward_noalloc: device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(HAD_ERR_UNSUPPORTED, "had_forward_noalloc: device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess)
      return failf(HAD_ERR_HIP, "had_forward_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return failf(HAD_ERR_HIP, "had_forward_noalloc: hipSetDevice: %s", hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr)
      return failf(HAD_ERR_HIP, "had_forward_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return HAD_OK;
}

}  // namespace
}  // namespace had

extern "C" had_status had_forward_noalloc(const float* q, const float* k, const void* v,
                                          had_dtype v_dtype, had_shape s, int64_t topn, float scale,
                                          int causal, uint32_t* qbits, uint32_t* kbits, float* out,
                                          float* sigma_q, float* sigma_k, uint32_t* dev_status,
                                          void* stream) {
  clear_error();
  had_status st = check_shape(s);
  if (st != HAD_OK) return st;
  const size_t need = had_forward_workspace_bytes(s);
  if (need > kScratchBytes)
    return failf(HAD_ERR_UNSUPPORTED, "had_forward_noalloc: needs %zu bytes of scratch, above the %zu-byte limit",
                 need, kScratchBytes);
  // every argument check runs before the scratch address is looked up
  if ((st = check_pack_args(q, qbits, sigma_q, "had_forward_noalloc")) != HAD_OK) return st;
  if ((st = check_pack_args(k, kbits, sigma_k, "had_forward_noalloc")) != HAD_OK) return st;
  if (dev_status != nullptr && !aligned(dev_status, 4))
    return fail(HAD_ERR_INVALID_ARG, "had_forward_noalloc: dev_status must be 4-byte aligned");
  AttnArgs unused;
  const int vdt = enum_bits(v_dtype);
  if ((st = attend_args(qbits, kbits, v, vdt, s, topn, scale, causal, out, "had_forward_noalloc", unused)) !=
      HAD_OK)
    return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (sigma_q != nullptr || sigma_k != nullptr) {
    if ((st = scratch_address(hs, &ws)) != HAD_OK) return st;
  }
  return forward_launch(q, k, v, vdt, s, topn, scale, causal, qbits, kbits, out, sigma_q, sigma_k,
                        static_cast<double*>(ws), dev_status, hs, "had_forward_noalloc");
}

extern "C" had_status had_select(const uint32_t* qbits, const uint32_t* kbits, had_shape s,
                                 int64_t topn, int causal, int64_t bh_begin, int64_t bh_count,
                                 int32_t* idx, void* stream) {
  clear_error();
  had_status st = check_shape(s);
  if (st != HAD_OK) return st;
  if ((st = check_bits(qbits, kbits, "had_select")) != HAD_OK) return st;
  if (idx == nullptr || !aligned(idx, 4)) return fail(HAD_ERR_INVALID_ARG, "had_select: null or unaligned idx");
  if (topn < 1) return fail(HAD_ERR_INVALID_ARG, "had_select: topn must be >= 1");
  if (topn > HAD_MAX_SEQ) return fail(HAD_ERR_UNSUPPORTED, "had_select: topn above HAD_MAX_SEQ");
  if (causal != 0 && causal != 1) return fail(HAD_ERR_INVALID_ARG, "had_select: causal must be 0 or 1");
  const int64_t bh_total = s.batch * s.heads;
  if (bh_begin < 0 || bh_count < 1 || bh_begin + bh_count > bh_total)
    return fail(HAD_ERR_INVALID_ARG, "had_select: bh range outside [0, B*H)");
  AttnArgs a{};
  a.qbits = qbits;
  a.kbits = kbits;
  a.v_dtype = HAD_BF16;
  a.bh_total = bh_total;
  a.bh_begin = bh_begin;
  a.bh_count = bh_count;
  a.n = static_cast<int>(s.seq);
  a.d = static_cast<int>(s.dim);
  a.topn = static_cast<int>(topn);
  a.causal = causal;
  a.idx = idx;
  return launch_attention_family(AttnMode::Select, a, static_cast<hipStream_t>(stream));
}

extern "C" had_status had_topn_mass(const uint32_t* qbits, const uint32_t* kbits, had_shape s,
                                    float scale, int causal, double mass, int64_t bh_begin,
                                    int64_t bh_count, int32_t* n_out, void* stream) {
  clear_error();
  had_status st = check_shape(s);
  if (st != HAD_OK) return st;
  if ((st = check_bits(qbits, kbits, "had_topn_mass")) != HAD_OK) return st;
  if (n_out == nullptr || !aligned(n_out, 4)) return fail(HAD_ERR_INVALID_ARG, "had_topn_mass: null or unaligned n_out");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(HAD_ERR_INVALID_ARG, "had_topn_mass: scale must be finite and > 0");
  if (!(mass > 0.0) || !std::isfinite(mass)) return fail(HAD_ERR_INVALID_ARG, "had_topn_mass: mass must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(HAD_ERR_INVALID_ARG, "had_topn_mass: causal must be 0 or 1");
  const int64_t bh_total = s.batch * s.heads;
  if (bh_begin < 0 || bh_count < 1 || bh_begin + bh_count > bh_total)
    return fail(HAD_ERR_INVALID_ARG, "had_topn_mass: bh range outside [0, B*H)");
  AttnArgs a{};
  a.qbits = qbits;
  a.kbits = kbits;
  a.v_dtype = HAD_BF16;
  a.bh_total = bh_total;
  a.bh_begin = bh_begin;
  a.bh_count = bh_count;
  a.n = static_cast<int>(s.seq);
  a.d = static_cast<int>(s.dim);
  a.topn = 1;
  a.scale = scale;
  a.causal = causal;
  a.mass = mass;
  a.nmass = n_out;
  return launch_attention_family(AttnMode::Mass, a, static_cast<hipStream_t>(stream));
}

extern "C" had_status had_logits(const uint32_t* qbits, const uint32_t* kbits, had_shape s,
                                 int64_t bh_begin, int64_t bh_count, int64_t row_begin,
                                 int64_t row_count, int16_t* s_out, void* stream) {
  clear_error();
  had_status st = check_shape(s);
  if (st != HAD_OK) return st;
  if ((st = check_bits(qbits, kbits, "had_logits")) != HAD_OK) return st;
  if (s_out == nullptr || !aligned(s_out, 2))
    return fail(HAD_ERR_INVALID_ARG, "had_logits: null or unaligned s_out");
  const int64_t bh_total = s.batch * s.heads;
  if (bh_begin < 0 || bh_count < 1 || bh_begin + bh_count > bh_total)
    return fail(HAD_ERR_INVALID_ARG, "had_logits: bh range outside [0, B*H)");
  if (row_begin < 0 || row_count < 1 || row_begin + row_count > s.seq)
    return fail(HAD_ERR_INVALID_ARG, "had_logits: row range outside [0, n)");
  AttnArgs a{};
  a.qbits = qbits;
  a.kbits = kbits;
  a.v_dtype = HAD_BF16;
  a.bh_total = bh_total;
  a.bh_begin = bh_begin;
  a.bh_count = bh_count;
  a.n = static_cast<int>(s.seq);
  a.d = static_cast<int>(s.dim);
  a.row_begin = static_cast<int>(row_begin);
  a.row_count = static_cast<int>(row_count);
  a.logits = s_out;
  return launch_attention_family(AttnMode::Logits, a, static_cast<hipStream_t>(stream));
}
