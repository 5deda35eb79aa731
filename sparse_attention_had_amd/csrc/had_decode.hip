// had_decode: HAD attention of a few new query rows against a long cache of
// packed keys and full-precision values (the decoding step of long-context
// inference).
//
// Method: the same path as had_attention (Pith review of "Hamming Attention
// Distillation", section "What carries the argument"; referee major comment 3
// for the full-precision values): integer logits s = d - 2h from the Hamming
// distance h of the sign words, the N_i largest visible logits of each row
// (lower key index wins among equal logits), softmax over that set and the
// weighted sum of the kept V rows.  Query i sits at position q_pos0 + i; with
// causal masking it sees keys j <= q_pos0 + i.
//
// GPU design.  With n_q << n_k the work is a scan of the key cache, so it is
// split over (key range, slice) work-groups and runs in four launches:
//  1. dec_hist: per split, h of every (query, key) pair by XOR + popcount on
//     the vector ALU (the query words are wave-uniform scalars), written as
//     16-bit values (0xFFFF for keys the row cannot see), and a per-split
//     (d+1)-bin histogram per query built with LDS atomics.
//  2. dec_stats: one wave per row sums the split histograms, finds the
//     threshold bin T and the tie quota r (as in had_attention), hands each
//     split its share of the r ties in split order (lower keys first), and
//     computes the softmax denominator Z from the counts.
//  3. dec_gather: per split and row, a wave walks the split's keys in order,
//     keeps h < T and the first quota keys with h == T (ballot ranks), and
//     reads only the kept V rows (2d bytes each for bf16, coalesced across
//     the wave), accumulating exp(-2*scale*(h - h_min)) * V_j in fp32.
//  4. dec_reduce: out = (sum over splits, in split order) / Z.
// HBM bytes per slice and row: the key words once (d/8 bytes per key, shared
// by the rows of a slice), 4 bytes per key for h, and 2d bytes per kept key.
#include <cmath>

#include "had_internal.h"

namespace had {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecQBatch = 16;        // rows per histogram work-group
constexpr int kDecMaxSplits = 512;
constexpr int kDecMinKeysPerSplit = 256;
constexpr uint32_t kDecHidden = 0xFFFFu;

struct DecArgs {
  const uint32_t* qbits;  // [BH, nq, W]
  const uint32_t* kbits;  // [BH, kstride, W]
  const void* v;          // [BH, kstride, d]
  int vf32;
  int64_t bh_total;
  int nq, nk, kstride, d, W;
  int64_t qpos0;
  int topn;
  float scale;
  int causal;
  float* out;             // [BH, nq, d]
  uint16_t* hbuf;         // [BH, nq, nk_pad]
  uint32_t* hist;         // [BH, nq, splits, d + 1]
  uint32_t* quota;        // [BH, nq, splits]
  int32_t* stats;         // [BH, nq, 4]: T, h_min, Z bits, N_i
  float* part;            // [BH, nq, splits, d]
  int splits;
  int keys_per_split;
  int nk_pad;
};

__device__ inline int visible_keys(const DecArgs& a, int q) {
  if (!a.causal) return a.nk;
  const int64_t last = a.qpos0 + q;  // the row sees keys 0 .. last
  return static_cast<int>(last + 1 < a.nk ? last + 1 : a.nk);
}

// ---- 1. logits and per-split histograms -------------------------------------
template <int W>
__global__ __launch_bounds__(kDecThreads) void dec_hist_kernel(DecArgs a) {
  __shared__ uint32_t hl[kDecQBatch * (HAD_MAX_DIM + 1)];
  const int nqb = (a.nq + kDecQBatch - 1) / kDecQBatch;
  const int64_t bid = blockIdx.x;
  const int s = static_cast<int>(bid % a.splits);
  const int qb = static_cast<int>((bid / a.splits) % nqb);
  const int64_t bh = bid / (static_cast<int64_t>(a.splits) * nqb);
  const int q0 = qb * kDecQBatch;
  const int nqh = min(kDecQBatch, a.nq - q0);
  const int nb = a.d + 1;
  const int k0 = s * a.keys_per_split;
  const int k1 = min(a.nk, k0 + a.keys_per_split);
  for (int t = threadIdx.x; t < nqh * nb; t += kDecThreads) hl[t] = 0u;
  __syncthreads();
  const uint32_t* qrow = a.qbits + (bh * a.nq + q0) * W;
  for (int jb = k0; jb < k0 + a.keys_per_split && jb < a.nk_pad; jb += kDecThreads) {
    const int j = jb + static_cast<int>(threadIdx.x);
    const bool valid = j < k1;
    uint32_t kw[W];
    const uint32_t* krow = a.kbits + (bh * a.kstride + (valid ? j : 0)) * W;
#pragma unroll
    for (int w = 0; w < W; ++w) kw[w] = valid ? krow[w] : 0u;
    for (int q = 0; q < nqh; ++q) {
      uint32_t h = 0;
#pragma unroll
      for (int w = 0; w < W; ++w) h += __builtin_popcount(kw[w] ^ qrow[q * W + w]);
      const bool vis = valid && (!a.causal || j <= a.qpos0 + q0 + q);
      if (j < a.nk_pad) a.hbuf[(bh * a.nq + q0 + q) * a.nk_pad + j] = static_cast<uint16_t>(vis ? h : kDecHidden);
      if (vis) atomicAdd(&hl[q * nb + h], 1u);
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < nqh * nb; t += kDecThreads) {
    const int q = t / nb, b = t - q * nb;
    a.hist[((bh * a.nq + q0 + q) * a.splits + s) * nb + b] = hl[t];
  }
}

// Inclusive prefix sum over the 64 lanes of a wave (integers: any order is exact).
__device__ inline uint32_t wave_scan_incl(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// ---- 2. per-row threshold, tie quotas and normalizer ------------------------
__global__ __launch_bounds__(64) void dec_stats_kernel(DecArgs a) {
  const int64_t bhq = blockIdx.x;
  const int q = static_cast<int>(bhq % a.nq);
  const int lane = threadIdx.x & 63;
  const int nb = a.d + 1;
  const uint32_t* hp = a.hist + bhq * a.splits * nb;
  const int Ni = min(a.topn, visible_keys(a, q));
  constexpr int kR = (HAD_MAX_DIM + 1 + 63) / 64;
  uint32_t cnt[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int b = 64 * r + lane;
    uint32_t c = 0;
    if (b < nb)
      for (int s = 0; s < a.splits; ++s) c += hp[s * nb + b];
    cnt[r] = c;
  }
  // threshold bin T: first bin whose inclusive count reaches N_i; h_min: first
  // non-empty bin
  int T = -1, hmin = -1;
  uint32_t below = 0, run = 0;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const uint32_t incl = wave_scan_incl(cnt[r]) + run;
    const uint32_t excl = incl - cnt[r];
    const bool hit = 64 * r + lane < nb && excl < static_cast<uint32_t>(Ni) && incl >= static_cast<uint32_t>(Ni);
    const uint64_t hm = __ballot(hit);
    if (T < 0 && hm != 0) {
      const int l = __builtin_ctzll(hm);
      T = 64 * r + l;
      below = __shfl(excl, l, 64);
    }
    const uint64_t nz = __ballot(64 * r + lane < nb && cnt[r] > 0);
    if (hmin < 0 && nz != 0) hmin = 64 * r + __builtin_ctzll(nz);
    run = __shfl(incl, 63, 64);
  }
  if (T < 0) T = a.d;  // unreachable: the visible count is >= N_i
  if (hmin < 0) hmin = 0;
  const uint32_t rtie = static_cast<uint32_t>(Ni) - below;
  // Z = sum_{b < T} cnt_b w(b - h_min) + r w(T - h_min), w(t) = exp(-2 scale t)
  double z = 0.0;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int b = 64 * r + lane;
    const uint32_t c = b < T ? cnt[r] : (b == T ? rtie : 0u);
    if (c != 0) z += static_cast<double>(c) * static_cast<double>(expf(-2.0f * a.scale * static_cast<float>(b - hmin)));
  }
  z = wave_sum_f64(z);  // total in lane 63, fixed order
  // the r ties go to the splits in key order
  uint32_t before = 0;
  for (int s0 = 0; s0 < a.splits; s0 += 64) {
    const int s = s0 + lane;
    const uint32_t tie = s < a.splits ? hp[s * nb + T] : 0u;
    const uint32_t incl = wave_scan_incl(tie) + before;
    const uint32_t excl = incl - tie;
    if (s < a.splits) {
      const uint32_t left = rtie > excl ? rtie - excl : 0u;
      a.quota[bhq * a.splits + s] = left < tie ? left : tie;
    }
    before = __shfl(incl, 63, 64);
  }
  if (lane == 63) {
    int32_t* st = a.stats + bhq * 4;
    st[0] = T;
    st[1] = hmin;
    st[2] = __builtin_bit_cast(int32_t, static_cast<float>(z));
    st[3] = Ni;
  }
}

// ---- 3. selection and gather of the kept V rows, per split ------------------
template <int F, bool VF32>
__global__ __launch_bounds__(kDecThreads) void dec_gather_kernel(DecArgs a) {
  const int64_t bid = blockIdx.x;
  const int s = static_cast<int>(bid % a.splits);
  const int64_t bh = bid / a.splits;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int k0 = s * a.keys_per_split;
  const int k1 = min(a.nk, k0 + a.keys_per_split);
  const int d = a.d;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int q = wid; q < a.nq; q += kDecThreads / 64) {
    const int64_t bhq = bh * a.nq + q;
    const int32_t* st = a.stats + bhq * 4;
    const uint32_t T = static_cast<uint32_t>(st[0]);
    const int hmin = st[1];
    const uint32_t quota = a.quota[bhq * a.splits + s];
    const uint16_t* hrow = a.hbuf + bhq * a.nk_pad;
    float acc[F];
#pragma unroll
    for (int f = 0; f < F; ++f) acc[f] = 0.0f;
    uint32_t tc = 0;  // ties of this row seen so far in this split
    for (int j0 = k0; j0 < k1; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t h = j < k1 ? hrow[j] : kDecHidden;
      const uint64_t tm = __ballot(h == T);
      const uint32_t rank = tc + static_cast<uint32_t>(__builtin_popcountll(tm & lt_mask));
      const bool keep = h < T || (h == T && rank < quota);
      tc += static_cast<uint32_t>(__builtin_popcountll(tm));
      const float wgt = keep ? expf(-2.0f * a.scale * static_cast<float>(static_cast<int>(h) - hmin)) : 0.0f;
      uint64_t km = __ballot(keep);
      // gather the kept rows, four in flight
      while (km != 0) {
        int jj[4];
        float ww[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (km != 0) {
            const int l = __builtin_ctzll(km);
            km &= km - 1;
            jj[u] = __builtin_amdgcn_readlane(j, l);
            ww[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wgt), l));
          } else {
            jj[u] = k0;
            ww[u] = 0.0f;
          }
        }
        float vv[4][F];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t row = (bh * a.kstride + jj[u]) * static_cast<int64_t>(d);
#pragma unroll
          for (int f = 0; f < F; ++f) {
            const int c = lane * F + f;
            if (VF32) {
              vv[u][f] = c < d ? static_cast<const float*>(a.v)[row + c] : 0.0f;
            } else {
              const uint16_t b = c < d ? static_cast<const uint16_t*>(a.v)[row + c] : 0;
              vv[u][f] = __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int f = 0; f < F; ++f) acc[f] = fmaf(ww[u], vv[u][f], acc[f]);
      }
    }
    float* prow = a.part + (bhq * a.splits + s) * static_cast<int64_t>(d);
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int c = lane * F + f;
      if (c < d) prow[c] = acc[f];
    }
  }
}

// ---- 4. fixed-order sum over splits, normalized ------------------------------
__global__ __launch_bounds__(64) void dec_reduce_kernel(DecArgs a) {
  const int64_t bhq = blockIdx.x;
  const float Z = __builtin_bit_cast(float, a.stats[bhq * 4 + 2]);
  const float invZ = Z > 0.0f ? 1.0f / Z : 0.0f;
  const float* p = a.part + bhq * a.splits * static_cast<int64_t>(a.d);
  for (int c = threadIdx.x; c < a.d; c += 64) {
    float sum = 0.0f;
    for (int s = 0; s < a.splits; ++s) sum += p[s * static_cast<int64_t>(a.d) + c];
    a.out[bhq * a.d + c] = sum * invZ;
  }
}

// Work split and workspace layout, from the shape alone.
struct DecPlan {
  int splits, keys_per_split, nk_pad;
  size_t off_h, off_hist, off_quota, off_stats, off_part, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

DecPlan plan_for(const had_decode_shape& s) {
  DecPlan p{};
  const int64_t bh = s.batch * s.heads;
  const int64_t nk = s.n_k;
  int64_t splits = (2048 + bh - 1) / bh;                 // aim at >= 2048 work-groups
  const int64_t max_by_keys = (nk + kDecMinKeysPerSplit - 1) / kDecMinKeysPerSplit;
  if (splits > max_by_keys) splits = max_by_keys;
  if (splits > kDecMaxSplits) splits = kDecMaxSplits;
  if (splits < 1) splits = 1;
  int64_t per = (nk + splits - 1) / splits;
  per = (per + 255) / 256 * 256;
  splits = (nk + per - 1) / per;
  p.splits = static_cast<int>(splits);
  p.keys_per_split = static_cast<int>(per);
  p.nk_pad = static_cast<int>((nk + 3) / 4 * 4);
  const size_t rows = static_cast<size_t>(bh) * static_cast<size_t>(s.n_q);
  size_t off = 0;
  p.off_h = off;
  off = align256(off + rows * p.nk_pad * sizeof(uint16_t));
  p.off_hist = off;
  off = align256(off + rows * p.splits * (s.dim + 1) * sizeof(uint32_t));
  p.off_quota = off;
  off = align256(off + rows * p.splits * sizeof(uint32_t));
  p.off_stats = off;
  off = align256(off + rows * 4 * sizeof(int32_t));
  p.off_part = off;
  off = align256(off + rows * p.splits * s.dim * sizeof(float));
  p.bytes = off;
  return p;
}

had_status check_decode_shape(const had_decode_shape& s) {
  if (s.batch <= 0 || s.heads <= 0 || s.n_q <= 0 || s.n_k <= 0 || s.dim <= 0)
    return fail(HAD_ERR_INVALID_ARG, "had_decode: shape fields must all be positive");
  if (s.k_stride < s.n_k) return fail(HAD_ERR_INVALID_ARG, "had_decode: k_stride must be >= n_k");
  if (s.dim > HAD_MAX_DIM) return fail(HAD_ERR_UNSUPPORTED, "had_decode: dim above HAD_MAX_DIM (256)");
  if (s.n_q > HAD_MAX_DECODE_Q) return fail(HAD_ERR_UNSUPPORTED, "had_decode: n_q above HAD_MAX_DECODE_Q");
  if (s.k_stride > HAD_MAX_DECODE_KEYS)
    return fail(HAD_ERR_UNSUPPORTED, "had_decode: k_stride above HAD_MAX_DECODE_KEYS");
  if (static_cast<double>(s.batch) * s.heads * s.n_q > 1.0e9)
    return fail(HAD_ERR_UNSUPPORTED, "had_decode: batch*heads*n_q too large");
  return HAD_OK;
}

template <int W>
void launch_hist(const DecArgs& a, int64_t blocks, hipStream_t st) {
  dec_hist_kernel<W><<<static_cast<unsigned>(blocks), kDecThreads, 0, st>>>(a);
}

template <int F>
void launch_gather(const DecArgs& a, int64_t blocks, hipStream_t st) {
  if (a.vf32)
    dec_gather_kernel<F, true><<<static_cast<unsigned>(blocks), kDecThreads, 0, st>>>(a);
  else
    dec_gather_kernel<F, false><<<static_cast<unsigned>(blocks), kDecThreads, 0, st>>>(a);
}

}  // namespace
}  // namespace had

using namespace had;

extern "C" size_t had_decode_workspace_bytes(had_decode_shape s) {
  if (check_decode_shape(s) != HAD_OK) return 0;
  return plan_for(s).bytes;
}

extern "C" had_status had_decode(const uint32_t* qbits, const uint32_t* kbits, const void* v,
                                 had_dtype v_dtype, had_decode_shape s, int64_t q_pos0,
                                 int64_t topn, float scale, int causal, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  had_status st = check_decode_shape(s);
  if (st != HAD_OK) return st;
  if (qbits == nullptr || kbits == nullptr || v == nullptr || out == nullptr)
    return fail(HAD_ERR_INVALID_ARG, "had_decode: null qbits, kbits, v or out");
  if (!aligned(qbits, 4) || !aligned(kbits, 4) || !aligned(v, 4) || !aligned(out, 4))
    return fail(HAD_ERR_INVALID_ARG, "had_decode: qbits, kbits, v and out must be 4-byte aligned");
  if (v_dtype != HAD_F32 && v_dtype != HAD_BF16) return fail(HAD_ERR_INVALID_ARG, "had_decode: unknown v_dtype");
  if (topn < 1) return fail(HAD_ERR_INVALID_ARG, "had_decode: topn must be >= 1");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(HAD_ERR_INVALID_ARG, "had_decode: scale must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(HAD_ERR_INVALID_ARG, "had_decode: causal must be 0 or 1");
  if (q_pos0 < 0 || q_pos0 > HAD_MAX_DECODE_KEYS)
    return fail(HAD_ERR_INVALID_ARG, "had_decode: q_pos0 must be in [0, HAD_MAX_DECODE_KEYS]");
  const DecPlan p = plan_for(s);
  if (workspace == nullptr || !aligned(workspace, 256))
    return fail(HAD_ERR_INVALID_ARG, "had_decode: workspace must be non-null and 256-byte aligned");
  if (workspace_bytes < p.bytes)
    return fail(HAD_ERR_INVALID_ARG, "had_decode: workspace smaller than had_decode_workspace_bytes()");
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  DecArgs a{};
  a.qbits = qbits;
  a.kbits = kbits;
  a.v = v;
  a.vf32 = v_dtype == HAD_F32;
  a.bh_total = s.batch * s.heads;
  a.nq = static_cast<int>(s.n_q);
  a.nk = static_cast<int>(s.n_k);
  a.kstride = static_cast<int>(s.k_stride);
  a.d = static_cast<int>(s.dim);
  a.W = static_cast<int>(words_per_row(s.dim));
  a.qpos0 = q_pos0;
  a.topn = static_cast<int>(topn > s.n_k ? s.n_k : topn);
  a.scale = scale;
  a.causal = causal;
  a.out = out;
  a.hbuf = reinterpret_cast<uint16_t*>(ws + p.off_h);
  a.hist = reinterpret_cast<uint32_t*>(ws + p.off_hist);
  a.quota = reinterpret_cast<uint32_t*>(ws + p.off_quota);
  a.stats = reinterpret_cast<int32_t*>(ws + p.off_stats);
  a.part = reinterpret_cast<float*>(ws + p.off_part);
  a.splits = p.splits;
  a.keys_per_split = p.keys_per_split;
  a.nk_pad = p.nk_pad;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int64_t nqb = (s.n_q + kDecQBatch - 1) / kDecQBatch;
  const int64_t hist_blocks = a.bh_total * nqb * p.splits;
  const int64_t gather_blocks = a.bh_total * p.splits;
  const int64_t rows = a.bh_total * s.n_q;
  if (hist_blocks > 0x7FFFFFFF || gather_blocks > 0x7FFFFFFF || rows > 0x7FFFFFFF)
    return fail(HAD_ERR_UNSUPPORTED, "had_decode: grid too large");
  switch (a.W) {
    case 1: launch_hist<1>(a, hist_blocks, hs); break;
    case 2: launch_hist<2>(a, hist_blocks, hs); break;
    case 3: launch_hist<3>(a, hist_blocks, hs); break;
    case 4: launch_hist<4>(a, hist_blocks, hs); break;
    case 5: launch_hist<5>(a, hist_blocks, hs); break;
    case 6: launch_hist<6>(a, hist_blocks, hs); break;
    case 7: launch_hist<7>(a, hist_blocks, hs); break;
    default: launch_hist<8>(a, hist_blocks, hs); break;
  }
  if ((st = check_launch("had_decode")) != HAD_OK) return st;
  dec_stats_kernel<<<static_cast<unsigned>(rows), 64, 0, hs>>>(a);
  if ((st = check_launch("had_decode")) != HAD_OK) return st;
  if (a.d <= 64)
    launch_gather<1>(a, gather_blocks, hs);
  else if (a.d <= 128)
    launch_gather<2>(a, gather_blocks, hs);
  else
    launch_gather<4>(a, gather_blocks, hs);
  if ((st = check_launch("had_decode")) != HAD_OK) return st;
  dec_reduce_kernel<<<static_cast<unsigned>(rows), 64, 0, hs>>>(a);
  return check_launch("had_decode");
}
