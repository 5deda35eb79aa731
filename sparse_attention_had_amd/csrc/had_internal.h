// Internal declarations shared by the HIP translation units of libhad.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "had.h"

namespace had {

// Thread-local text of the last failure (returned by had_last_error()).
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

inline had_status fail(had_status st, const char* what) {
  set_error("%s", what);
  return st;
}
had_status failf(had_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

inline had_status check_launch(const char* kernel) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s launch failed: %s", kernel, hipGetErrorString(e));
    return HAD_ERR_HIP;
  }
  return HAD_OK;
}

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

inline int64_t words_per_row(int64_t d) { return (d + 31) / 32; }

// The int a C caller passed for an enum parameter, read as bytes: a value
// outside the enum's range must be rejected, not loaded as the enum type.
template <typename E>
inline int enum_bits(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  memcpy(&v, &e, sizeof(v));
  return v;
}
inline bool valid_dtype(int v) { return v == HAD_F32 || v == HAD_BF16; }

// Shape checks common to every entry point; seq may not exceed max_seq
// (HAD_MAX_SEQ for the attention calls, the cache limit for had_pack).
had_status check_shape(const had_shape& s, int64_t max_seq = HAD_MAX_SEQ);

// ---- pack (had_pack.hip) ----
constexpr int kPackThreads = 256;    // threads per pack block
// Pack blocks per tensor, at most.  256 blocks x 4 waves, each with two
// batches of 4 KiB of loads in flight, keep about 64 KiB of reads in flight
// per CU on a fused Q+K launch: a measured optimum for streaming fp32 Q and
// K (twice that or half of it is 5-10 % slower).
constexpr int kPackMaxBlocks = 256;
constexpr int kPackWavesPerBlock = kPackThreads / 64;

int pack_grid_blocks(const had_shape& s);
// Sigma partial pairs (sum x, sum x^2) a pack launch writes per tensor: one
// per block, at most kPackMaxBlocks.
int pack_partials(const had_shape& s);

// One tensor of a pack launch.
struct PackJob {
  const float* x;
  uint32_t* bits;
  double* partials;  // 2 doubles per pack block, or null (no sigma)
};

had_status check_pack_args(const float* x, uint32_t* xbits, float* sigma, const char* who);
// Packs njobs (1 or 2) tensors of shape s; one launch when the two can share it.
had_status launch_pack(const PackJob* jobs, int njobs, const had_shape& s, uint32_t* dev_status,
                       hipStream_t st);
// One-wave kernel: sigma from the partials of a pack launch of shape s.
had_status launch_sigma_finalize(const double* partials, const had_shape& s, float* sigma,
                                 hipStream_t st);

// v + (the value DPP control kCtrl brings to this lane, 0.0 where the row
// mask leaves a lane out), on the two 32-bit halves of a double.
template <int kCtrl, int kRowMask>
__device__ inline double dpp_add_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u), kCtrl, kRowMask, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), kCtrl, kRowMask, 0xF, false);
  const uint64_t w = (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
  return v + __builtin_bit_cast(double, w);
}

// Wave sum of a double in a fixed order (neighbour pairs, quads, rows of 16,
// then across rows); lane 63 holds the total, the same on every run.
__device__ inline double wave_sum_f64(double v) {
  v = dpp_add_f64<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add_f64<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add_f64<0x124, 0xF>(v);  // row_ror:4
  v = dpp_add_f64<0x128, 0xF>(v);  // row_ror:8
  v = dpp_add_f64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add_f64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// One wave (lanes 0..63 of the calling wave): totals of the nparts partial
// pairs (sum x, sum x^2) in a fixed order.  Lane l sums partials l, l + 64,
// ... in order (eight loads in flight), then a fixed-order wave sum; the
// totals are valid in lane 63.
__device__ inline void partials_total(const double2* partials, int nparts, double& a, double& b) {
  constexpr int kBatch = 8;
  const int lane = threadIdx.x & 63;
  a = 0.0;
  b = 0.0;
  for (int base = 0; base < nparts; base += 64 * kBatch) {
    double2 p[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = base + lane + 64 * k;
      p[k] = i < nparts ? partials[i] : double2{0.0, 0.0};
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      a += p[k].x;
      b += p[k].y;
    }
  }
  a = wave_sum_f64(a);
  b = wave_sum_f64(b);
}

// One wave: lane 63 writes the population standard deviation of count
// elements from the partial pairs of their pack launch.
__device__ inline void sigma_from_partials(const double2* partials, int nparts, double count,
                                           float* sigma) {
  double a, b;
  partials_total(partials, nparts, a, b);
  if ((threadIdx.x & 63) == 63) {
    const double mean = a / count;
    double var = b / count - mean * mean;
    if (!(var > 0.0)) var = 0.0;
    *sigma = static_cast<float>(sqrt(var));
  }
}

// ---- attention family (had_attention.hip) ----
enum class AttnMode : int { Attend = 0, Select = 1, Logits = 2, Mass = 3, Stats = 4 };

struct AttnArgs {
  const uint32_t* qbits;
  const uint32_t* kbits;
  const void* v;
  had_dtype v_dtype;
  int64_t bh_total;  // B*H
  int64_t bh_begin;  // first (batch, head) slice processed
  int64_t bh_count;  // slices processed
  int n;             // tokens per slice
  int d;             // features
  int topn;          // N (Select / Attend)
  float scale;       // softmax scale (Attend)
  int causal;        // 0/1
  int row_begin;     // first query row processed (Logits)
  int row_count;     // query rows processed (Logits)
  float* out;        // Attend output [bh_total, n, d]
  int32_t* idx;      // Select output [bh_count, n, topn]
  int16_t* logits;   // Logits output [bh_count, row_count, n]
  double mass;       // Mass: softmax mass to reach
  int32_t* nmass;    // Mass output [bh_count, n]
  // Stats output [bh_count, n, 4]: threshold bin T, index of the last kept key
  // whose logit sits at the threshold (-1 if none), h_min, and Z (float bits)
  // = the sum over the kept keys of exp(-2*scale*(h - h_min))
  int32_t* rowstats;
  // Build option HAD_FUSED_QPACK (a measurement build): the attend launch
  // reads float32 Q rows itself, stores their sign words in qbits_out and
  // one (sum, sum of squares) pair per wave in qpartials for sigma_Q.
  const float* qf;
  int qf_vec;          // rows 16-byte aligned and d a multiple of 32: vector loads
  uint32_t* qbits_out;
  double* qpartials;
  uint32_t* dev_status;
  int balance;       // set by the launcher: the whole grid is resident at once
  // Optional sigma finalize (fused forward call): wave 0 of the last block
  // turns the partials of a preceding pack launch into sigma_out[t].
  const double2* sigma_partials[2];
  float* sigma_out[2];
  int sigma_nparts;
  double sigma_count;
};

had_status launch_attention_family(AttnMode mode, const AttnArgs& a, hipStream_t st);
// Waves one attend launch of shape s runs (the per-wave sigma partials of
// the HAD_FUSED_QPACK build).
int64_t attend_wave_count(const had_shape& s);
// One wave: sigma from nparts partial pairs of count elements.
had_status launch_sigma_finalize_n(const double* partials, int64_t nparts, double count, float* sigma,
                                   hipStream_t st);

}  // namespace had
