// had_pack: standardize + sign-binarize + bit-pack of Q or K, plus sigma.
//
// Method (Pith review of "Hamming Attention Distillation", section "What
// carries the argument"; referee minor comment 6 on Eq. 12): Q and K are
// divided by a data-estimated standard deviation over all elements of the
// matrix and passed through sign().  Dividing by sigma > 0 never changes a
// sign, so the bit of element x is simply [x < 0] and sigma is a separate
// reduction reported to the caller.
//
// Data path (HBM-bound, one read of x):
//  * d % 32 == 0: the rows are contiguous, so the flat element stream maps
//    onto the flat word stream (word = element / 32).  With x 16-byte
//    aligned, lane L of a wave loads floats 4L..4L+3 of a 256-float segment;
//    the 8 lanes that cover one word OR their sign nibbles together and one
//    of them stores the word.  Each wave owns a contiguous run of segments
//    (runs differ by at most one segment) and keeps up to kUnroll 1 KiB loads
//    in flight.  Unaligned x falls back to one 64-float ballot per load.
//  * other d: one thread per output word (pad bits stay 0).
//  * sigma: every thread sums x and x*x in float64; blocks reduce in a fixed
//    order and store one partial pair each to the workspace; a one-block
//    finalize kernel on the same stream sums the partials in index order and
//    writes sigma.  (A "last block finalizes" scheme needs an agent-scope
//    release per block, which writes back L2 and costs more than the whole
//    pack.)  No floating-point atomics, so sigma is bit-identical from run to
//    run.
#include "had_internal.h"

namespace had {
namespace {

constexpr int kPackThreads = 256;
constexpr int kPackMaxBlocks = 1024;
constexpr int kUnroll = 8;
constexpr int kSegsPerWave = 4;  // grid sizing target for small inputs

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Block-level fixed-order sum of two doubles; result valid in thread 0.
__device__ inline void block_sum2(double& a, double& b) {
  __shared__ double red[2][kPackThreads / 64];
  a = wave_sum(a);
  b = wave_sum(b);
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wid] = a;
    red[1][wid] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a = 0.0;
    b = 0.0;
    for (int w = 0; w < kPackThreads / 64; ++w) {
      a += red[0][w];
      b += red[1][w];
    }
  }
}

// Per-block partial sums (plain stores; the finalize kernel that follows on
// the same stream sees them through kernel-boundary ordering).
__device__ void write_partials(double s1, double s2, double* partials) {
  block_sum2(s1, s2);
  if (threadIdx.x == 0) {
    partials[2 * blockIdx.x + 0] = s1;
    partials[2 * blockIdx.x + 1] = s2;
  }
}

// One block: sum the partials in a fixed order and write sigma.  Thread t
// owns partials t, t + 256, ...; all of its loads are issued before the sum.
__global__ __launch_bounds__(kPackThreads) void sigma_finalize_kernel(const double2* partials,
                                                                       int nblocks, double count,
                                                                       float* sigma) {
  constexpr int kPer = kPackMaxBlocks / kPackThreads;
  double2 p[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = threadIdx.x + k * kPackThreads;
    p[k] = i < nblocks ? partials[i] : double2{0.0, 0.0};
  }
  double a = 0.0, b = 0.0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    a += p[k].x;
    b += p[k].y;
  }
  block_sum2(a, b);
  if (threadIdx.x == 0) {
    const double mean = a / count;
    double var = b / count - mean * mean;
    if (!(var > 0.0)) var = 0.0;
    *sigma = static_cast<float>(sqrt(var));
  }
}

// d % 32 == 0 and x 16-byte aligned: 256-float segments, 8 words each.
template <bool kSigma>
__global__ __launch_bounds__(kPackThreads) void pack_vec_kernel(
    const f32x4* __restrict__ x, uint32_t* __restrict__ bits, int64_t elems, double* partials,
    uint32_t* dev_status) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kPackThreads + threadIdx.x) >> 6;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kPackThreads / 64);
  const int64_t nseg = (elems + 255) >> 8;
  const int64_t seg_end = (wave + 1) * nseg / nwaves;
  const int64_t nvec = elems >> 2;
  const int64_t nwords = elems >> 5;
  const int shift = 4 * (lane & 7);
  double s1 = 0.0, s2 = 0.0;
  bool nan_seen = false;
  for (int64_t s0 = wave * nseg / nwaves; s0 < seg_end; s0 += kUnroll) {
    f32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = (s0 + u) * 64 + lane;
      v[u] = (s0 + u < seg_end && i < nvec) ? __builtin_nontemporal_load(x + i)
                                            : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const f32x4 e = v[u];
      uint32_t w = (static_cast<uint32_t>(e.x < 0.0f) | (static_cast<uint32_t>(e.y < 0.0f) << 1) |
                    (static_cast<uint32_t>(e.z < 0.0f) << 2) |
                    (static_cast<uint32_t>(e.w < 0.0f) << 3))
                   << shift;
      w |= __shfl_xor(w, 1, 64);
      w |= __shfl_xor(w, 2, 64);
      w |= __shfl_xor(w, 4, 64);
      const int64_t wi = (s0 + u) * 8 + (lane >> 3);
      if ((lane & 7) == 0 && s0 + u < seg_end && wi < nwords) bits[wi] = w;
      nan_seen |= (e.x != e.x) | (e.y != e.y) | (e.z != e.z) | (e.w != e.w);
      if (kSigma) {
        const double a = e.x, b = e.y, c = e.z, d = e.w;
        s1 += (a + b) + (c + d);
        s2 += fma(a, a, b * b) + fma(c, c, d * d);
      }
    }
  }
  if (dev_status != nullptr && __ballot(nan_seen) != 0 && lane == 0)
    atomicOr(dev_status, HAD_DEV_NAN_INPUT);
  if (kSigma) write_partials(s1, s2, partials);
}

// d % 32 == 0, x not 16-byte aligned: 64 elements -> 2 words per ballot.
template <bool kSigma>
__global__ __launch_bounds__(kPackThreads) void pack_stream_kernel(
    const float* __restrict__ x, uint32_t* __restrict__ bits, int64_t elems, double* partials,
    uint32_t* dev_status) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kPackThreads + threadIdx.x) >> 6;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kPackThreads / 64);
  const int64_t nchunks = (elems + 63) >> 6;
  const int64_t nwords = elems >> 5;
  double s1 = 0.0, s2 = 0.0;
  bool nan_seen = false;
  for (int64_t c0 = wave * kUnroll; c0 < nchunks; c0 += nwaves * kUnroll) {
    float v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t e = (c0 + u) * 64 + lane;
      v[u] = (e < elems) ? __builtin_nontemporal_load(x + e) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t m = __ballot(v[u] < 0.0f);
      nan_seen |= (v[u] != v[u]);
      if (kSigma) {
        const double dv = static_cast<double>(v[u]);
        s1 += dv;
        s2 = fma(dv, dv, s2);
      }
      const int64_t w = (c0 + u) * 2 + lane;
      if (lane < 2 && w < nwords) bits[w] = static_cast<uint32_t>(m >> (32 * lane));
    }
  }
  if (dev_status != nullptr && __ballot(nan_seen) != 0 && lane == 0)
    atomicOr(dev_status, HAD_DEV_NAN_INPUT);
  if (kSigma) write_partials(s1, s2, partials);
}

// Any d: one thread per output word.
template <bool kSigma>
__global__ __launch_bounds__(kPackThreads) void pack_rows_kernel(
    const float* __restrict__ x, uint32_t* __restrict__ bits, int64_t rows, int d, int W,
    double* partials, uint32_t* dev_status) {
  const int64_t nwords = rows * W;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kPackThreads;
  double s1 = 0.0, s2 = 0.0;
  bool nan_seen = false;
  for (int64_t wi = static_cast<int64_t>(blockIdx.x) * kPackThreads + threadIdx.x; wi < nwords;
       wi += stride) {
    const int64_t r = wi / W;
    const int w = static_cast<int>(wi - r * W);
    const float* row = x + r * d;
    const int c_end = min(d, 32 * w + 32);
    uint32_t word = 0;
    for (int c = 32 * w; c < c_end; ++c) {
      const float v = row[c];
      word |= static_cast<uint32_t>(v < 0.0f) << (c - 32 * w);
      nan_seen |= (v != v);
      if (kSigma) {
        const double dv = static_cast<double>(v);
        s1 += dv;
        s2 = fma(dv, dv, s2);
      }
    }
    bits[wi] = word;
  }
  if (dev_status != nullptr && __ballot(nan_seen) != 0 && (threadIdx.x & 63) == 0)
    atomicOr(dev_status, HAD_DEV_NAN_INPUT);
  if (kSigma) write_partials(s1, s2, partials);
}

}  // namespace

int pack_grid_blocks(const had_shape& s) {
  const int64_t elems = s.batch * s.heads * s.seq * s.dim;
  int64_t blocks;
  if (s.dim % 32 == 0) {
    const int64_t segs = (elems + 255) / 256;
    const int64_t waves = (segs + kSegsPerWave - 1) / kSegsPerWave;
    blocks = (waves + kPackThreads / 64 - 1) / (kPackThreads / 64);
  } else {
    const int64_t words = s.batch * s.heads * s.seq * words_per_row(s.dim);
    blocks = (words + kPackThreads - 1) / kPackThreads;
  }
  if (blocks < 1) blocks = 1;
  if (blocks > kPackMaxBlocks) blocks = kPackMaxBlocks;
  return static_cast<int>(blocks);
}

}  // namespace had

using namespace had;

extern "C" size_t had_pack_workspace_bytes(had_shape s) {
  if (check_shape(s) != HAD_OK) return 0;
  return sizeof(double) * 2 * static_cast<size_t>(pack_grid_blocks(s));
}

extern "C" had_status had_pack(const float* x, had_shape s, uint32_t* xbits, float* sigma,
                               void* workspace, size_t workspace_bytes, uint32_t* dev_status,
                               void* stream) {
  clear_error();
  had_status st = check_shape(s);
  if (st != HAD_OK) return st;
  if (x == nullptr || xbits == nullptr) return fail(HAD_ERR_INVALID_ARG, "had_pack: null x or xbits");
  if (!aligned(x, 4) || !aligned(xbits, 4))
    return fail(HAD_ERR_INVALID_ARG, "had_pack: x and xbits must be 4-byte aligned");
  if (dev_status != nullptr && !aligned(dev_status, 4))
    return fail(HAD_ERR_INVALID_ARG, "had_pack: dev_status must be 4-byte aligned");
  const int blocks = pack_grid_blocks(s);
  double* partials = nullptr;
  if (sigma != nullptr) {
    if (!aligned(sigma, 4)) return fail(HAD_ERR_INVALID_ARG, "had_pack: sigma must be 4-byte aligned");
    if (workspace == nullptr || !aligned(workspace, 16))
      return fail(HAD_ERR_INVALID_ARG, "had_pack: sigma requested but workspace is null or unaligned");
    if (workspace_bytes < had_pack_workspace_bytes(s))
      return fail(HAD_ERR_INVALID_ARG, "had_pack: workspace smaller than had_pack_workspace_bytes()");
    partials = static_cast<double*>(workspace);
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int64_t rows = s.batch * s.heads * s.seq;
  const int d = static_cast<int>(s.dim);
  if (d % 32 == 0) {
    const int64_t elems = rows * d;
    const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
    if (aligned(x, 16) && sigma)
      pack_vec_kernel<true><<<blocks, kPackThreads, 0, hs>>>(x4, xbits, elems, partials, dev_status);
    else if (aligned(x, 16))
      pack_vec_kernel<false><<<blocks, kPackThreads, 0, hs>>>(x4, xbits, elems, nullptr, dev_status);
    else if (sigma)
      pack_stream_kernel<true><<<blocks, kPackThreads, 0, hs>>>(x, xbits, elems, partials, dev_status);
    else
      pack_stream_kernel<false><<<blocks, kPackThreads, 0, hs>>>(x, xbits, elems, nullptr, dev_status);
  } else {
    const int W = static_cast<int>(words_per_row(d));
    if (sigma)
      pack_rows_kernel<true><<<blocks, kPackThreads, 0, hs>>>(x, xbits, rows, d, W, partials, dev_status);
    else
      pack_rows_kernel<false><<<blocks, kPackThreads, 0, hs>>>(x, xbits, rows, d, W, nullptr, dev_status);
  }
  had_status ls = check_launch("had_pack");
  if (ls != HAD_OK || sigma == nullptr) return ls;
  sigma_finalize_kernel<<<1, kPackThreads, 0, hs>>>(reinterpret_cast<const double2*>(partials), blocks, static_cast<double>(rows) * d, sigma);
  return check_launch("had_pack");
}
