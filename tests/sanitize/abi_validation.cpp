// Host-side validation of the libhad C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point is called with arguments that
// its checks must reject before any GPU work, and must return the documented
// status with an error text.  The library's C++ is compiled for the host only
// (no device code), so this runs without a GPU; nothing here launches a
// kernel.  Exit status 0 means every check held and the sanitizers found
// nothing.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "had.h"

static int g_fail = 0;

static void expect(had_status got, had_status want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, want %d\n", what, static_cast<int>(got), static_cast<int>(want));
    ++g_fail;
    return;
  }
  if (got != HAD_OK && had_last_error()[0] == '\0') {
    std::fprintf(stderr, "FAIL %s: no error text\n", what);
    ++g_fail;
  }
}

#define EXPECT(call, want) expect((call), (want), #call)

// Fake, never-dereferenced device addresses (16-byte aligned unless offset).
static void* A(uintptr_t a) { return reinterpret_cast<void*>(a); }
template <typename T>
static T* P(uintptr_t a) { return reinterpret_cast<T*>(a); }

int main() {
  const had_shape ok{1, 2, 128, 64};
  const had_shape zero{1, 0, 128, 64};
  const had_shape bigd{1, 2, 128, 257};
  const had_shape bign{1, 2, 70000, 64};
  const had_shape huge{1 << 30, 1 << 30, 1 << 30, 256};
  const float nan = std::numeric_limits<float>::quiet_NaN();

  // sizes and strings
  if (had_words_per_row(0) != 0 || had_words_per_row(33) != 2 || had_words_per_row(256) != 8) ++g_fail;
  if (had_pack_workspace_bytes(zero) != 0 || had_pack_workspace_bytes(huge) != 0) ++g_fail;
  if (had_forward_workspace_bytes(huge) != 0 || had_backward_workspace_bytes(bigd) != 0) ++g_fail;
  for (int st = -1; st < 6; ++st)
    if (had_status_string(static_cast<had_status>(st)) == nullptr) ++g_fail;

  // had_pack
  const size_t pws = had_pack_workspace_bytes(ok);
  EXPECT(had_pack(nullptr, ok, P<uint32_t>(0x2000), nullptr, nullptr, 0, nullptr, nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_pack(P<float>(0x1002), ok, P<uint32_t>(0x2000), nullptr, nullptr, 0, nullptr, nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_pack(P<float>(0x1000), ok, P<uint32_t>(0x2000), P<float>(0x3000), nullptr, pws, nullptr, nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_pack(P<float>(0x1000), ok, P<uint32_t>(0x2000), P<float>(0x3000), A(0x4000), pws - 1, nullptr, nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_pack(P<float>(0x1000), zero, P<uint32_t>(0x2000), nullptr, nullptr, 0, nullptr, nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_pack(P<float>(0x1000), bigd, P<uint32_t>(0x2000), nullptr, nullptr, 0, nullptr, nullptr), HAD_ERR_UNSUPPORTED);
  EXPECT(had_pack(P<float>(0x1000), huge, P<uint32_t>(0x2000), nullptr, nullptr, 0, nullptr, nullptr), HAD_ERR_UNSUPPORTED);
  EXPECT(had_pack(P<float>(0x1000), ok, P<uint32_t>(0x2000), nullptr, nullptr, 0, P<uint32_t>(0x5002), nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_pack_calibrate(P<float>(0x1000), ok, P<uint32_t>(0x2000), nullptr, A(0x4000), pws, nullptr, nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_sigma_from_state(nullptr, P<float>(0x1000), nullptr), HAD_ERR_INVALID_ARG);

  // had_attention
  auto attn = [&](const uint32_t* q, const void* v, int dt, had_shape s, int64_t topn, float scale, int causal, float* out) {
    return had_attention(q, P<uint32_t>(0x2000), v, static_cast<had_dtype>(dt), s, topn, scale, causal, out, nullptr);
  };
  EXPECT(attn(nullptr, A(0x3000), 1, ok, 8, 0.1f, 0, P<float>(0x4000)), HAD_ERR_INVALID_ARG);
  EXPECT(attn(P<uint32_t>(0x1000), A(0x3004), 1, ok, 8, 0.1f, 0, P<float>(0x4000)), HAD_ERR_INVALID_ARG);
  EXPECT(attn(P<uint32_t>(0x1000), A(0x3000), 7, ok, 8, 0.1f, 0, P<float>(0x4000)), HAD_ERR_INVALID_ARG);
  EXPECT(attn(P<uint32_t>(0x1000), A(0x3000), 1, ok, 0, 0.1f, 0, P<float>(0x4000)), HAD_ERR_INVALID_ARG);
  EXPECT(attn(P<uint32_t>(0x1000), A(0x3000), 1, ok, 8, nan, 0, P<float>(0x4000)), HAD_ERR_INVALID_ARG);
  EXPECT(attn(P<uint32_t>(0x1000), A(0x3000), 1, ok, 8, -1.0f, 0, P<float>(0x4000)), HAD_ERR_INVALID_ARG);
  EXPECT(attn(P<uint32_t>(0x1000), A(0x3000), 1, ok, 8, 0.1f, 2, P<float>(0x4000)), HAD_ERR_INVALID_ARG);
  EXPECT(attn(P<uint32_t>(0x1000), A(0x3000), 1, bign, 8, 0.1f, 0, P<float>(0x4000)), HAD_ERR_UNSUPPORTED);
  EXPECT(attn(P<uint32_t>(0x1000), A(0x3000), 1, huge, 8, 0.1f, 0, P<float>(0x4000)), HAD_ERR_UNSUPPORTED);

  // had_forward and had_forward_noalloc
  const size_t fws = had_forward_workspace_bytes(ok);
  EXPECT(had_forward(P<float>(0x1000), P<float>(0x1100), A(0x3000), HAD_BF16, ok, 8, 0.1f, 0, P<uint32_t>(0x5000),
                     P<uint32_t>(0x6000), P<float>(0x4000), P<float>(0x7000), nullptr, A(0x8000), fws - 1, nullptr,
                     nullptr),
         HAD_ERR_INVALID_ARG);
  EXPECT(had_forward(nullptr, P<float>(0x1100), A(0x3000), HAD_BF16, ok, 8, 0.1f, 0, P<uint32_t>(0x5000),
                     P<uint32_t>(0x6000), P<float>(0x4000), nullptr, nullptr, nullptr, 0, nullptr, nullptr),
         HAD_ERR_INVALID_ARG);
  EXPECT(had_forward_noalloc(P<float>(0x1000), P<float>(0x1100), A(0x3000), HAD_BF16, ok, 8, 0.1f, 0,
                             P<uint32_t>(0x5000), nullptr, P<float>(0x4000), P<float>(0x7000), nullptr, nullptr,
                             nullptr),
         HAD_ERR_INVALID_ARG);
  EXPECT(had_forward_noalloc(P<float>(0x1000), P<float>(0x1100), A(0x3000), HAD_BF16, bign, 8, 0.1f, 0,
                             P<uint32_t>(0x5000), P<uint32_t>(0x6000), P<float>(0x4000), nullptr, nullptr, nullptr,
                             nullptr),
         HAD_ERR_UNSUPPORTED);

  // inspection exports and the top-N mass
  EXPECT(had_logits(P<uint32_t>(0x1000), P<uint32_t>(0x2000), ok, 0, 3, 0, 10, P<int16_t>(0x3000), nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_logits(P<uint32_t>(0x1000), P<uint32_t>(0x2000), ok, 0, 2, 120, 10, P<int16_t>(0x3000), nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_select(P<uint32_t>(0x1000), P<uint32_t>(0x2000), ok, 0, 0, 0, 2, P<int32_t>(0x3000), nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_select(P<uint32_t>(0x1000), P<uint32_t>(0x2000), ok, 70000, 0, 0, 2, P<int32_t>(0x3000), nullptr), HAD_ERR_UNSUPPORTED);
  EXPECT(had_select(P<uint32_t>(0x1000), P<uint32_t>(0x2000), ok, 8, 0, -1, 2, P<int32_t>(0x3000), nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_topn_mass(P<uint32_t>(0x1000), P<uint32_t>(0x2000), ok, 0.1f, 0, 1e300 * 1e300, 0, 2, P<int32_t>(0x3000), nullptr), HAD_ERR_INVALID_ARG);
  EXPECT(had_topn_mass(P<uint32_t>(0x1000), P<uint32_t>(0x2000), ok, 0.1f, 0, 0.9, 0, 2, nullptr, nullptr), HAD_ERR_INVALID_ARG);

  // had_decode and had_decode_forward
  const had_decode_shape ds{1, 2, 4, 1000, 1024, 64};
  const size_t dws = had_decode_workspace_bytes(ds);
  const had_decode_shape dbad{1, 2, 4, 1000, 999, 64};
  const had_decode_shape dbig{1, 2, HAD_MAX_DECODE_Q + 1, 1000, 1024, 64};
  if (dws == 0 || had_decode_workspace_bytes(dbad) != 0) ++g_fail;
  EXPECT(had_decode(P<uint32_t>(0x1000), P<uint32_t>(0x2000), A(0x3000), HAD_BF16, ds, 996, 8, 0.1f, 1, P<float>(0x4000),
                    A(0x10000), dws - 1, nullptr),
         HAD_ERR_INVALID_ARG);
  EXPECT(had_decode(P<uint32_t>(0x1000), P<uint32_t>(0x2000), A(0x3000), HAD_BF16, dbad, 996, 8, 0.1f, 1, P<float>(0x4000),
                    A(0x10000), dws, nullptr),
         HAD_ERR_INVALID_ARG);
  EXPECT(had_decode(P<uint32_t>(0x1000), P<uint32_t>(0x2000), A(0x3000), HAD_BF16, dbig, 996, 8, 0.1f, 1, P<float>(0x4000),
                    A(0x10000), dws, nullptr),
         HAD_ERR_UNSUPPORTED);
  EXPECT(had_decode(P<uint32_t>(0x1000), P<uint32_t>(0x2000), A(0x3000), HAD_BF16, ds, -1, 8, 0.1f, 1, P<float>(0x4000),
                    A(0x10000), dws, nullptr),
         HAD_ERR_INVALID_ARG);
  EXPECT(had_decode_forward(nullptr, P<uint32_t>(0x2000), A(0x3000), HAD_BF16, ds, 996, 8, 0.1f, 1, P<float>(0x4000),
                            A(0x10000), dws, nullptr),
         HAD_ERR_INVALID_ARG);

  // had_backward
  const size_t bws = had_backward_workspace_bytes(ok);
  EXPECT(had_backward(P<uint32_t>(0x1000), P<uint32_t>(0x2000), A(0x3000), HAD_BF16, ok, 8, 0.1f, 0, P<float>(0x4000),
                      P<float>(0x5000), nullptr, nullptr, P<float>(0x6000), P<float>(0x7000), P<float>(0x8000),
                      A(0x10000), bws - 1, nullptr),
         HAD_ERR_INVALID_ARG);
  EXPECT(had_backward(P<uint32_t>(0x1000), P<uint32_t>(0x2000), A(0x3000), HAD_BF16, bigd, 8, 0.1f, 0, P<float>(0x4000),
                      P<float>(0x5000), nullptr, nullptr, P<float>(0x6000), P<float>(0x7000), P<float>(0x8000),
                      A(0x10000), bws, nullptr),
         HAD_ERR_UNSUPPORTED);
  EXPECT(had_backward(P<uint32_t>(0x1000), P<uint32_t>(0x2000), A(0x3000), HAD_BF16, ok, 8, 0.1f, 0, nullptr,
                      P<float>(0x5000), nullptr, nullptr, P<float>(0x6000), P<float>(0x7000), P<float>(0x8000),
                      A(0x10000), bws, nullptr),
         HAD_ERR_INVALID_ARG);

  // had_soft_forward / had_soft_select
  const had_shape soft_long = {1, 2, 1025, 64};
  if (had_soft_workspace_bytes(soft_long) != 0 || had_soft_workspace_bytes(bigd) != 0) ++g_fail;
  const size_t sws = had_soft_workspace_bytes(ok);
  EXPECT(had_soft_forward(P<float>(0x1000), P<float>(0x2000), A(0x3000), HAD_BF16, ok, 8, 0.1f, 0.5f, 0, nullptr,
                          nullptr, P<float>(0x4000), A(0x10000), sws - 1, nullptr),
         HAD_ERR_INVALID_ARG);
  EXPECT(had_soft_forward(P<float>(0x1000), P<float>(0x2000), A(0x3000), HAD_BF16, ok, 8, 0.1f, 0.0f, 0, nullptr,
                          nullptr, P<float>(0x4000), A(0x10000), sws, nullptr),
         HAD_ERR_INVALID_ARG);
  EXPECT(had_soft_forward(P<float>(0x1000), P<float>(0x2000), A(0x3000), static_cast<had_dtype>(7), ok, 8, 0.1f,
                          0.5f, 0, nullptr, nullptr, P<float>(0x4000), A(0x10000), sws, nullptr),
         HAD_ERR_INVALID_ARG);
  EXPECT(had_soft_forward(P<float>(0x1000), P<float>(0x2000), A(0x3000), HAD_BF16, soft_long, 8, 0.1f, 0.5f, 0,
                          nullptr, nullptr, P<float>(0x4000), A(0x10000), sws, nullptr),
         HAD_ERR_UNSUPPORTED);
  EXPECT(had_soft_select(P<float>(0x1000), P<float>(0x2000), ok, 8, 0.5f, 0, nullptr, nullptr, 0, 0,
                         P<uint8_t>(0x4000), A(0x10000), sws, nullptr),
         HAD_ERR_INVALID_ARG);
  EXPECT(had_soft_select(P<float>(0x1000), P<float>(0x2000), ok, 8, 0.5f, 0, nullptr, nullptr, 0, 1, nullptr,
                         A(0x10000), sws, nullptr),
         HAD_ERR_INVALID_ARG);

  if (g_fail == 0) std::printf("abi validation: all checks held\n");
  return g_fail == 0 ? 0 : 1;
}
