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
// split over (key range, slice) work-groups (256 * 2^m keys per split, at
// most 2048) and runs in three launches:
//  1. dec_hist: per split and batch of up to 16 rows, h of every (row, key)
//     pair by XOR + popcount on the vector ALU (the query words are
//     wave-uniform scalars; key rows as vector loads) into a per-split
//     (d+1)-bin histogram per row (LDS atomics).  With n_q <= W it also
//     stores h of every (row, key) as one byte ("bins").
//  2. dec_gather: one 256-thread work-group per (split, row).  Its keys'
//     distances are requested first (the bins, or the key words again,
//     L2-resident after step 1), and meanwhile wave 0 sums the row's split
//     histograms, finds the threshold bin T and the tie quota r (as in
//     had_attention) and this split's share of the r ties (lower splits
//     first); the split-0 work-group also writes the softmax denominator Z.
//     h < T and the first quota keys with h == T are kept in key order (wave
//     ballots plus one work-group prefix over (key step, wave) counts), the
//     kept keys and their distances are compacted in LDS, and only the kept
//     V rows are read, 16 bytes of a row per lane, with weights
//     exp(-2*scale*(h - h_min)) from a table, accumulating in fp32; the row
//     groups are summed in a fixed order.
//  3. dec_reduce: out = (sum over splits, in split order) / Z.
// HBM bytes per slice: the key words (d/8 bytes per key), and per row the
// 2d bytes (bf16) of each kept key; everything else is small.
#include <atomic>
#include <cmath>

#include "had_internal.h"

namespace had {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecQBatch = 16;           // rows per histogram work-group
constexpr int kDecMaxSplits = 2048;
constexpr int kDecMinKeysPerSplit = 256;
constexpr int kDecMaxKeysPerSplit = 2048;

struct DecArgs {
  const uint32_t* qbits;  // [BH, nq, W] (had_decode_forward: written by the histogram launch)
  const float* qf;        // [BH, nq, d] float32 new rows (had_decode_forward), else null
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
  uint8_t* bins;          // [BH, nq, nkp] Hamming distance of every (row, key), or null
  int64_t nkp;            // bins row length (splits * keys_per_split)
  uint32_t* hist;         // [BH, nq, splits, d + 1]
  int32_t* stats;         // [BH, nq, 4]: T, h_min, Z bits, N_i
  float* part;            // [BH, nq, splits, d]
  int splits;
  int keys_per_split;
  int fparts;             // single-launch path: work-groups per (slice, row), each for 1/fparts of the columns
};

__device__ inline int visible_keys(const DecArgs& a, int q) {
  if (!a.causal) return a.nk;
  const int64_t last = a.qpos0 + q;  // the row sees keys 0 .. last
  return static_cast<int>(last + 1 < a.nk ? last + 1 : a.nk);
}

// Key words of one key: W dwords, as vector loads where the row alignment
// allows (kKVec: the cache base is 16-byte aligned for W % 4 == 0, 8-byte
// aligned for W % 2 == 0).
template <int W, bool kKVec>
__device__ inline void load_key_words(const uint32_t* krow, uint32_t* kw) {
  if constexpr (kKVec && W % 4 == 0) {
#pragma unroll
    for (int w = 0; w < W; w += 4) {
      const uint4 t = *reinterpret_cast<const uint4*>(krow + w);
      kw[w] = t.x; kw[w + 1] = t.y; kw[w + 2] = t.z; kw[w + 3] = t.w;
    }
  } else if constexpr (kKVec && W % 2 == 0) {
#pragma unroll
    for (int w = 0; w < W; w += 2) {
      const uint2 t = *reinterpret_cast<const uint2*>(krow + w);
      kw[w] = t.x; kw[w + 1] = t.y;
    }
  } else {
#pragma unroll
    for (int w = 0; w < W; ++w) kw[w] = krow[w];
  }
}

// ---- 1. logits and per-split histograms -------------------------------------
// kQF: the new rows arrive as float32 (had_decode_forward); each work-group
// builds their sign words itself (bit c of word w is [x_{32w+c} < 0], pad bits
// 0, as had_pack), and the split-0 work-groups store them for the gather.
template <int W, bool kKVec, bool kQF>
__global__ __launch_bounds__(kDecThreads) void dec_hist_kernel(DecArgs a) {
  __shared__ uint32_t hl[kDecQBatch * (HAD_MAX_DIM + 1)];
  __shared__ uint32_t qs[kQF ? kDecQBatch * W : 1];
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
  const uint32_t* qrow = kQF ? qs : a.qbits + (bh * a.nq + q0) * W;
  constexpr int kU = 4;  // keys per thread in flight
  uint32_t kw[kU][W];
  int j[kU];
  auto load = [&](int jb) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      j[u] = jb + u * kDecThreads + static_cast<int>(threadIdx.x);
      load_key_words<W, kKVec>(a.kbits + (bh * a.kstride + (j[u] < k1 ? j[u] : 0)) * W, kw[u]);
    }
  };
  load(k0);  // the first keys are in flight while the histogram is cleared
  for (int t = threadIdx.x; t < nqh * nb; t += kDecThreads) hl[t] = 0u;
  if constexpr (kQF) {
    // wave w packs rows w, w + 4, ...: one ballot per 64 elements = 2 words
    const int lane = threadIdx.x & 63;
    for (int q = static_cast<int>(threadIdx.x >> 6); q < nqh; q += kDecThreads / 64) {
      const float* xr = a.qf + (bh * a.nq + q0 + q) * static_cast<int64_t>(a.d);
#pragma unroll
      for (int w2 = 0; w2 < W; w2 += 2) {
        const int e = 32 * w2 + lane;
        const uint64_t m = __ballot(e < a.d && xr[e < a.d ? e : 0] < 0.0f);
        if (lane < 2 && w2 + lane < W) {
          const uint32_t word = static_cast<uint32_t>(m >> (32 * lane));
          qs[q * W + w2 + lane] = word;
          if (s == 0) const_cast<uint32_t*>(a.qbits)[(bh * a.nq + q0 + q) * W + w2 + lane] = word;
        }
      }
    }
  }
  __syncthreads();
  for (int jb = k0; jb < k1; jb += kU * kDecThreads) {
    if (jb != k0) load(jb);
    for (int q = 0; q < nqh; ++q) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        uint32_t h = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) h += __builtin_popcount(kw[u][w] ^ qrow[q * W + w]);
        const bool vis = j[u] < k1 && (!a.causal || j[u] <= a.qpos0 + q0 + q);
        if (vis) atomicAdd(&hl[q * nb + h], 1u);
        if (a.bins != nullptr && j[u] < k1) a.bins[(bh * a.nq + q0 + q) * a.nkp + j[u]] = static_cast<uint8_t>(h);
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < nqh * nb; t += kDecThreads) {
    const int q = t / nb, b = t - q * nb;
    a.hist[((bh * a.nq + q0 + q) * a.splits + s) * nb + b] = hl[t];
  }
}

// x + (the value DPP control kCtrl brings to this lane; 0 where there is no
// source lane or the row mask leaves this lane out).
template <int kCtrl, int kRowMask>
__device__ inline uint32_t dpp_add_u32(uint32_t x) {
  return x + static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kCtrl, kRowMask, 0xF, true));
}

// Inclusive prefix sum over the 64 lanes of a wave on DPP lane moves: shifts
// by 1, 2, 4, 8 within rows of 16, then each row adds the last lane of the
// rows before it (integers: any order is exact).
__device__ inline uint32_t wave_scan_incl(uint32_t x) {
  x = dpp_add_u32<0x111, 0xF>(x);  // row_shr:1
  x = dpp_add_u32<0x112, 0xF>(x);  // row_shr:2
  x = dpp_add_u32<0x114, 0xF>(x);  // row_shr:4
  x = dpp_add_u32<0x118, 0xF>(x);  // row_shr:8
  x = dpp_add_u32<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_add_u32<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// ---- 2. per-row threshold, this split's tie quota and the normalizer ---------
// Run by one wave (lanes 0..63).  Sums the row's split histograms, finds the
// threshold bin T (the first bin whose count from h = 0 up reaches N_i) and
// h_min (the first non-empty bin), and gives split s_self its share of the
// r = N_i - (keys below T) ties: the ties of lower splits come first.  With
// write_stats, also writes T, h_min, Z and N_i for the final reduce.
struct RowStats {
  uint32_t T;
  int hmin;
  uint32_t quota;
};

template <int W>
__device__ RowStats row_stats(const DecArgs& a, int64_t bhq, int q, int s_self, bool write_stats) {
  const int lane = threadIdx.x & 63;
  const int nb = a.d + 1;
  const uint32_t* hp = a.hist + bhq * a.splits * nb;
  const int Ni = min(a.topn, visible_keys(a, q));
  constexpr int kR = (32 * W + 1 + 63) / 64;  // 64-bin rows of the d + 1 <= 32W + 1 bins
  uint32_t cnt[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) cnt[r] = 0u;
  // up to three rows of 8 splits in flight at once: one round trip per 8
  // splits for d < 192, two above (24 loads keep the gather at 8 waves per SIMD)
  constexpr int kRB = kR < 3 ? kR : 3;
#pragma unroll
  for (int r0 = 0; r0 < kR; r0 += kRB) {
    for (int s0 = 0; s0 < a.splits; s0 += 8) {
      uint32_t t[kRB][8];
#pragma unroll
      for (int r = 0; r < kRB; ++r) {
        const int b = 64 * (r0 + r) + lane;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          t[r][u] = (r0 + r < kR && b < nb && s0 + u < a.splits) ? hp[(s0 + u) * nb + b] : 0u;
      }
#pragma unroll
      for (int r = 0; r < kRB; ++r) {
        if (r0 + r < kR) {
#pragma unroll
          for (int u = 0; u < 8; ++u) cnt[r0 + r] += t[r][u];
        }
      }
    }
  }
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
      below = __builtin_amdgcn_readlane(excl, l);
    }
    const uint64_t nz = __ballot(64 * r + lane < nb && cnt[r] > 0);
    if (hmin < 0 && nz != 0) hmin = 64 * r + __builtin_ctzll(nz);
    run = __builtin_amdgcn_readlane(incl, 63);
  }
  if (T < 0) T = a.d;  // unreachable: the visible count is >= N_i
  if (hmin < 0) hmin = 0;
  const uint32_t rtie = static_cast<uint32_t>(Ni) - below;
  // ties at T in the splits before s_self
  uint32_t before = 0, mine = 0;
  for (int s0 = 0; s0 < a.splits; s0 += 64) {
    const int sp = s0 + lane;
    const uint32_t tie = sp < a.splits ? hp[sp * nb + T] : 0u;
    uint32_t x = sp < s_self ? tie : 0u;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    before += x;
    if (s_self >= s0 && s_self < s0 + 64) mine = __shfl(tie, s_self - s0, 64);
  }
  const uint32_t left = rtie > before ? rtie - before : 0u;
  RowStats rs{static_cast<uint32_t>(T), hmin, left < mine ? left : mine};
  if (write_stats) {
    // Z = sum_{b < T} cnt_b w(b - h_min) + r w(T - h_min), w(t) = exp(-2 scale t)
    double z = 0.0;
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int b = 64 * r + lane;
      const uint32_t c = b < T ? cnt[r] : (b == T ? rtie : 0u);
      if (c != 0) z += static_cast<double>(c) * static_cast<double>(expf(-2.0f * a.scale * static_cast<float>(b - hmin)));
    }
    z = wave_sum_f64(z);  // total in lane 63, fixed order
    if (lane == 63) {
      int32_t* st = a.stats + bhq * 4;
      st[0] = T;
      st[1] = hmin;
      st[2] = __builtin_bit_cast(int32_t, static_cast<float>(z));
      st[3] = Ni;
    }
  }
  return rs;
}

// ---- 3. selection and gather of the kept V rows, per (split, row) ------------
// Thread t owns the keys k0 + t + 256*u (u < kpt = keys_per_split / 256, a
// power of two <= 8), so key order is (u, wave, lane) and every load below
// is coalesced across the wave.  The Hamming distances come from the bins
// the histogram launch wrote (kBins: one byte per key) or are recomputed
// from the key words (kGrp keys per batch); either way the first loads are
// in flight while wave 0 computes the row statistics.  A kept key's slot in
// the list is (strict keys before it) + min(ties before it, quota), from
// per-(u, wave) ballot counts.  The list (key offset << 16 | h per entry)
// lives in dynamic LDS of keys_per_split dwords; the row-group partial sums
// reuse that space after the gather.  V rows are read 8 features per lane:
// kVec = 16-byte vector loads (bf16 with d % 8 == 0, or fp32 with d % 4 == 0,
// and a 16-byte aligned base), several rows per lane group in flight.
constexpr int kDecWaves = kDecThreads / 64;
constexpr int cmin(int x, int y) { return x < y ? x : y; }

size_t gather_lds_bytes(int keys_per_split) {
  const size_t list = static_cast<size_t>(keys_per_split) * 4;
  const size_t red = static_cast<size_t>(kDecThreads) * 8 * 4;
  return list > red ? list : red;
}

constexpr int kDecMaxKPT = kDecMaxKeysPerSplit / kDecThreads;  // keys per thread, at most

template <int W, bool VF32, bool kVec, bool kKVec, bool kBins>
__global__ __launch_bounds__(kDecThreads) void dec_gather_kernel(DecArgs a) {
  extern __shared__ uint32_t dyn[];  // list, then red
  __shared__ float wtab[HAD_MAX_DIM + 1];
  __shared__ uint32_t cnt[kDecMaxKPT][kDecWaves];  // strict | ties << 16, per (u, wave)
  __shared__ RowStats rs_sh;
  uint32_t* list = dyn;
  float* red = reinterpret_cast<float*>(dyn);
  const int64_t bid = blockIdx.x;
  const int s = static_cast<int>(bid % a.splits);
  const int64_t rest = bid / a.splits;
  const int q = static_cast<int>(rest % a.nq);
  const int64_t bh = rest / a.nq;
  const int64_t bhq = bh * a.nq + q;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int d = a.d;
  const int k0 = s * a.keys_per_split;
  const int k1 = min(a.nk, k0 + a.keys_per_split);
  const int64_t last = a.causal ? a.qpos0 + q : static_cast<int64_t>(a.nk);  // keys j <= last
  const int kend = static_cast<int>(min(static_cast<int64_t>(k1), last + 1));  // visible: [k0, kend)
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int kpt = a.keys_per_split / kDecThreads;  // wave-uniform

  // ---- Hamming distances of this thread's keys (meaningless where a key is
  // not visible; never used there)
  uint32_t hh[kDecMaxKPT];
  // keys per batch: about 16 key words in flight
  constexpr int kGrp = cmin(kDecMaxKPT, W <= 2 ? 8 : (W <= 4 ? 4 : 2));
  uint32_t kw[kBins ? 1 : kGrp][W];
  const uint32_t* qw = a.qbits + bhq * W;
  const uint32_t* kb = a.kbits + bh * static_cast<int64_t>(a.kstride) * W;
  auto load_batch = [&](int u0) {
    if constexpr (!kBins) {
#pragma unroll
      for (int g = 0; g < kGrp; ++g) {
        const int j = k0 + (u0 + g) * kDecThreads + tid;
        if (u0 + g < kpt && j < kend) {
          load_key_words<W, kKVec>(kb + static_cast<int64_t>(j) * W, kw[g]);
        } else {
#pragma unroll
          for (int w = 0; w < W; ++w) kw[g][w] = 0u;
        }
      }
    }
  };
  auto finish_batch = [&](int u0) {
    if constexpr (!kBins) {
#pragma unroll
      for (int g = 0; g < kGrp; ++g) {
        uint32_t h = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) h += __builtin_popcount(kw[g][w] ^ qw[w]);
        hh[u0 + g] = h;
      }
    }
  };
  if constexpr (kBins) {
    // one byte per key, 64 consecutive bytes per wave; the bins row holds
    // splits * keys_per_split entries, so every load stays inside it
    const uint8_t* brow = a.bins + bhq * a.nkp + k0 + tid;
#pragma unroll
    for (int u = 0; u < kDecMaxKPT; ++u) hh[u] = u < kpt ? brow[u * kDecThreads] : 0u;
  } else {
    load_batch(0);
  }
  for (int t = tid; t <= d; t += kDecThreads) wtab[t] = expf(-2.0f * a.scale * static_cast<float>(t));
  // the row's threshold and this split's tie quota (wave 0), shared through LDS
  if (wid == 0) {
    const RowStats r0 = row_stats<W>(a, bhq, q, s, s == 0);
    if (lane == 0) rs_sh = r0;
  }
  if constexpr (!kBins) {
    finish_batch(0);
#pragma unroll
    for (int u0 = kGrp; u0 < kDecMaxKPT; u0 += kGrp) {
      if (u0 < kpt) {
        load_batch(u0);
        finish_batch(u0);
      }
    }
  }
  __syncthreads();
  const uint32_t T = rs_sh.T;
  const int hmin = rs_sh.hmin;
  const uint32_t quota = rs_sh.quota;

  // ---- per-(u, wave) counts of strict keys (h < T) and ties (h == T),
  // packed as strict | ties << 16 (a split holds at most 2048 keys)
#pragma unroll
  for (int u = 0; u < kDecMaxKPT; ++u) {
    if (u >= kpt) break;
    const bool vis = k0 + u * kDecThreads + tid < kend;
    const uint64_t sm = __ballot(vis && hh[u] < T);
    const uint64_t tm = __ballot(vis && hh[u] == T);
    if (lane == 0)
      cnt[u][wid] = static_cast<uint32_t>(__builtin_popcountll(sm)) |
                    (static_cast<uint32_t>(__builtin_popcountll(tm)) << 16);
  }
  __syncthreads();
  // ---- ranks and the compacted list, in key order
  uint32_t run = 0;  // strict | ties << 16 in earlier u
#pragma unroll
  for (int u = 0; u < kDecMaxKPT; ++u) {
    if (u >= kpt) break;
    const int j = k0 + u * kDecThreads + tid;
    const bool vis = j < kend;
    const bool strict = vis && hh[u] < T;
    const bool tie = vis && hh[u] == T;
    const uint64_t sm = __ballot(strict);
    const uint64_t tm = __ballot(tie);
    uint32_t wb = 0, ut = 0;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const uint32_t c = cnt[u][w];
      wb += w < wid ? c : 0u;
      ut += c;
    }
    const uint32_t b = run + wb;
    const uint32_t sbefore = (b & 0xFFFFu) + static_cast<uint32_t>(__builtin_popcountll(sm & lt_mask));
    const uint32_t tbefore = (b >> 16) + static_cast<uint32_t>(__builtin_popcountll(tm & lt_mask));
    if (strict || (tie && tbefore < quota))
      list[sbefore + min(tbefore, quota)] = (static_cast<uint32_t>(j - k0) << 16) | hh[u];
    run += ut;
  }
  const int nl = static_cast<int>((run & 0xFFFFu) + min(run >> 16, quota));
  __syncthreads();  // the list is complete

  // ---- gather: lpr lanes per V row, 8 features each; R row groups
  const int lpr = (d + 7) / 8;
  const int R = kDecThreads / lpr;
  const int g = tid / lpr, li = tid - (tid / lpr) * lpr;
  float acc[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) acc[f] = 0.0f;
  const unsigned char* vbase = static_cast<const unsigned char*>(a.v) +
                               bh * static_cast<int64_t>(a.kstride) * d * (VF32 ? 4 : 2);
  constexpr int kRows = VF32 ? 4 : 6;  // rows per lane group in flight (<= 64 VGPRs for bf16)
  if (g < R) {
    const int c0 = 8 * li;
    for (int e0 = g; e0 < nl; e0 += kRows * R) {
      uint32_t raw[kRows][VF32 ? 8 : 4];
      float wr[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int e = e0 + r * R;
        const uint32_t ent = e < nl ? list[e] : list[e0];
        // (clamps keep every access inside the visible keys and the table)
        const int hb = min(max(static_cast<int>(ent & 0xFFFFu) - hmin, 0), d);
        wr[r] = e < nl ? wtab[hb] : 0.0f;
        const int64_t jj = min(k0 + static_cast<int>(ent >> 16), kend - 1);
        if constexpr (VF32) {
          const float* row = reinterpret_cast<const float*>(vbase) + jj * d;
          if (kVec && c0 + 8 <= d) {
            const uint4 u0 = *reinterpret_cast<const uint4*>(row + c0);
            const uint4 u1 = *reinterpret_cast<const uint4*>(row + c0 + 4);
            raw[r][0] = u0.x; raw[r][1] = u0.y; raw[r][2] = u0.z; raw[r][3] = u0.w;
            raw[r][4] = u1.x; raw[r][5] = u1.y; raw[r][6] = u1.z; raw[r][7] = u1.w;
          } else {
#pragma unroll
            for (int f = 0; f < 8; ++f) raw[r][f] = c0 + f < d ? __builtin_bit_cast(uint32_t, row[c0 + f]) : 0u;
          }
        } else {
          const uint16_t* row = reinterpret_cast<const uint16_t*>(vbase) + jj * d;
          if (kVec && c0 + 8 <= d) {
            const uint4 u = *reinterpret_cast<const uint4*>(row + c0);
            raw[r][0] = u.x; raw[r][1] = u.y; raw[r][2] = u.z; raw[r][3] = u.w;
          } else {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
              const uint32_t lo = c0 + 2 * f < d ? row[c0 + 2 * f] : 0u;
              const uint32_t hi = c0 + 2 * f + 1 < d ? row[c0 + 2 * f + 1] : 0u;
              raw[r][f] = lo | (hi << 16);
            }
          }
        }
      }
      // rows e0, e0 + R, ... in order (entries past nl have weight 0)
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        float x[8];
        if constexpr (VF32) {
#pragma unroll
          for (int f = 0; f < 8; ++f) x[f] = __builtin_bit_cast(float, raw[r][f]);
        } else {
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            x[2 * f] = __builtin_bit_cast(float, raw[r][f] << 16);
            x[2 * f + 1] = __builtin_bit_cast(float, raw[r][f] & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int f = 0; f < 8; ++f) acc[f] = fmaf(wr[r], x[f], acc[f]);
      }
    }
  }
  __syncthreads();  // every group is done with the list: red reuses it
  // row-group partial sums, then a fixed-order sum over the groups
  if (g < R) {
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int c = 8 * li + f;
      if (c < d) red[g * d + c] = acc[f];
    }
  }
  __syncthreads();
  float* prow = a.part + (bhq * a.splits + s) * static_cast<int64_t>(d);
  for (int c = tid; c < d; c += kDecThreads) {
    float sum = 0.0f;
    for (int gg = 0; gg < R; ++gg) sum += red[gg * d + c];
    prow[c] = sum;
  }
}

// ---- 4. fixed-order sum over splits, normalized ------------------------------
// One thread per feature (blockDim = d rounded up to 64), 16 loads in flight.
__global__ __launch_bounds__(HAD_MAX_DIM) void dec_reduce_kernel(DecArgs a) {
  const int64_t bhq = blockIdx.x;
  const int c = threadIdx.x;
  if (c >= a.d) return;
  const float Z = __builtin_bit_cast(float, a.stats[bhq * 4 + 2]);
  const float invZ = Z > 0.0f ? 1.0f / Z : 0.0f;
  const float* p = a.part + bhq * a.splits * static_cast<int64_t>(a.d) + c;
  constexpr int kB = 16;
  float sum = 0.0f;
  for (int s0 = 0; s0 < a.splits; s0 += kB) {  // summed in split order
    float t[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) t[u] = s0 + u < a.splits ? p[(s0 + u) * static_cast<int64_t>(a.d)] : 0.0f;
#pragma unroll
    for (int u = 0; u < kB; ++u) sum += t[u];
  }
  a.out[bhq * a.d + c] = sum * invZ;
}

// ---- single-launch path for few rows ---------------------------------------
// When there are few (slice, row) pairs (at most 4096, and at most 16 new
// rows per slice), each pair gets fparts 1024-thread work-groups that share
// out the feature columns: every one of them scans all of the row's keys (so
// each has the row's histogram, threshold, tie quota and kept list without
// any exchange), then gathers only its 1/fparts of each kept V row and writes
// those output columns.  No split histograms or partial outputs go through
// memory and there is no reduce launch.  fparts > 1 lets a few rows use every
// CU: gathering scattered V rows is limited by the loads a CU keeps in
// flight, so one work-group per row on half the CUs reaches little more than
// half the device rate.  The work-groups of a slice (or, with fewer than 8
// slices, of a pair) are placed on one XCD, so the repeated key scan and the
// shared V rows are served by that XCD's L2.
// Thread t owns keys t + 1024 u (u < 16, so at most 16384 keys); key order
// is (u, wave, lane) as in dec_gather.  Distances go to one LDS histogram;
// wave 0 finds T, h_min, the tie quota and Z from it; the distances, stored
// by key, are read back 16 consecutive keys per thread, and a thread's kept
// keys get their list slots from its counts, a scan over the threads and a
// walk in key order; the kept V rows are gathered 16 bytes of a row per lane
// with several rows in flight per lane group, and the row groups' sums are
// added in a fixed order and divided by Z.  The per-key steps are written
// for few vector instructions (hidden keys carry an out-of-range distance
// instead of a visibility test; slots come from per-thread counts rather than
// per-key ballots): each costs 4 cycles of a SIMD per wave, and the fparts
// copies of the scan and list repeat them.
constexpr int kOneThreads = 1024;
constexpr int kOneWaves = kOneThreads / 64;
constexpr int kOneKPT = 16;                              // keys per thread
constexpr int kOneMaxKeys = kOneThreads * kOneKPT;       // 16384
constexpr int kOneMaxList = 8192;                        // kept keys per row (LDS list)
constexpr int kOneMaxPairs = 4096;                       // (slice, row) pairs that take this path
constexpr int kOneMaxRows = 16;                          // new rows per slice that take this path

template <int W, bool VF32, bool kVec, bool kKVec, bool kQF>
__global__ __launch_bounds__(kOneThreads) __attribute__((amdgpu_waves_per_eu(4)))
void dec_one_kernel(DecArgs a) {
  __shared__ uint32_t hist[1024];  // the row's histogram (d + 1 bins); then the final partial sums
  __shared__ __attribute__((aligned(16))) uint32_t list[kOneMaxList];  // (key << 9) | (h - h_min) per kept key; then the row-group sums
  __shared__ float wtab[HAD_MAX_DIM + 1];
  __shared__ __attribute__((aligned(16))) uint32_t wtot[kOneWaves];  // per-wave strict | ties << 16
  __shared__ int sh_T, sh_hmin, sh_quota;
  __shared__ float sh_invz;
  float* red = reinterpret_cast<float*>(list);
  float* red2 = reinterpret_cast<float*>(hist);
  // With at least 8 slices, index = ((slice / 8) * nq * fparts + row * fparts
  // + part) * 8 + slice % 8: every row and part of a slice on one XCD
  // (work-groups are dealt to the XCDs round robin by index), so its key
  // words and kept V rows are shared in that XCD's L2.  With fewer slices,
  // index = ((pair / 8) * fparts + part) * 8 + pair % 8, so that the pairs
  // still spread over the XCDs (the parts of a pair stay together).
  const int P = a.fparts;
  const int rest = static_cast<int>(blockIdx.x >> 3);
  const int part = rest % P;
  const int r2 = rest / P;
  int q;
  int64_t bh, bhq;
  if (a.bh_total >= 8) {
    q = r2 % a.nq;
    bh = static_cast<int64_t>(r2 / a.nq) * 8 + (blockIdx.x & 7);
    if (bh >= a.bh_total) return;  // padding of the last group of 8 slices
    bhq = bh * a.nq + q;
  } else {
    bhq = static_cast<int64_t>(r2) * 8 + (blockIdx.x & 7);
    if (bhq >= a.bh_total * a.nq) return;  // padding of the last group of 8 pairs
    q = static_cast<int>(bhq % a.nq);
    bh = bhq / a.nq;
  }
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int d = a.d, nb = d + 1;
  const int64_t last = a.causal ? a.qpos0 + q : static_cast<int64_t>(a.nk) - 1;
  const int kend = static_cast<int>(min(static_cast<int64_t>(a.nk), last + 1));  // visible keys [0, kend)
  const int Ni = min(a.topn, kend);
  // this part's feature columns: 8-column slots [s0, s0 + ns) of the row's (d + 7) / 8
  const int slots = (d + 7) / 8;
  const int sp = (slots + P - 1) / P;
  const int s0 = part * sp;
  const int ns = min(sp, slots - s0);  // >= 1: the host picks fparts so that every part has a slot

  // this thread's keys, a batch of kG in flight at a time; the first batch is
  // requested before the row's sign words are ready.  The loads are
  // unconditional (keys past the visible end read the last visible key,
  // kend >= 1) and only the histogram update is predicated.
  const uint32_t* kb = a.kbits + bh * static_cast<int64_t>(a.kstride) * W;
  // 32 bytes of key words per lane per batch: at d = 128 (W = 4), 2 keys per
  // batch measured 21.1 us per decode, 1 key 22.6, 4 keys 21.6, 8 keys 22.0
  // and 16 keys 24.4 (fewer requests in flight per lane, staggered over the
  // batches, are served faster)
  constexpr int kG = W >= 5 ? 1 : (W >= 3 ? 2 : 8 / W);
  static_assert(kOneKPT % kG == 0, "whole batches");
  uint32_t kw[kG][W];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const int j = min(g * kOneThreads + tid, kend - 1);
    load_key_words<W, kKVec>(kb + static_cast<int64_t>(j) * W, kw[g]);
  }

  // the row's sign words, in every wave (wave-uniform): built from the
  // float32 row for had_decode_forward (bit c of word w is [x_{32w+c} < 0],
  // pad bits 0, as had_pack), else read; requested along with the keys
  uint32_t qw[W];
  constexpr int kQL = (W + 1) / 2;  // 64-element row chunks
  float qx[kQF ? kQL : 1];
  if constexpr (kQF) {
    const float* xr = a.qf + bhq * static_cast<int64_t>(d);
#pragma unroll
    for (int i = 0; i < kQL; ++i) {
      const int e = 64 * i + lane;
      qx[i] = xr[e < d ? e : 0];
    }
  } else {
#pragma unroll
    for (int w = 0; w < W; ++w) qw[w] = a.qbits[bhq * W + w];
  }
  for (int t = tid; t < nb; t += kOneThreads) hist[t] = 0u;
  for (int t = tid; t <= d; t += kOneThreads) wtab[t] = expf(-2.0f * a.scale * static_cast<float>(t));
  __syncthreads();
  if constexpr (kQF) {
#pragma unroll
    for (int i = 0; i < kQL; ++i) {
      const uint64_t m = __ballot(64 * i + lane < d && qx[i] < 0.0f);
      qw[2 * i] = static_cast<uint32_t>(m);
      if (2 * i + 1 < W) qw[2 * i + 1] = static_cast<uint32_t>(m >> 32);
    }
  }

  // distances into the row's LDS histogram (one for the work-group: same-bin
  // conflicts measured no slower than per-wave copies, and the threshold scan
  // reads one row), and every key's distance into the list's space as a
  // 16-bit value at the key's index (the list stage reads them back 16
  // consecutive keys per thread); a hidden key (past the visible end) keeps
  // the distance kHidden, above every threshold bin (T <= d)
  constexpr uint32_t kHidden = 0x1FFu;
  uint16_t* hkey = reinterpret_cast<uint16_t*>(list);
  uint32_t* hw = hist;
#pragma unroll
  for (int u0 = 0; u0 < kOneKPT; u0 += kG) {
    if (u0 > 0) {
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const int j = min((u0 + g) * kOneThreads + tid, kend - 1);
        load_key_words<W, kKVec>(kb + static_cast<int64_t>(j) * W, kw[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      uint32_t h = 0;
#pragma unroll
      for (int w = 0; w < W; ++w) h += __builtin_popcount(kw[g][w] ^ qw[w]);
      const bool vis = (u0 + g) * kOneThreads + tid < kend;
      hkey[(u0 + g) * kOneThreads + tid] = static_cast<uint16_t>(vis ? h : kHidden);
      if (vis) atomicAdd(&hw[h], 1u);
    }
  }
  __syncthreads();

  // wave 0: threshold bin T, h_min, tie quota r, Z
  if (wid == 0) {
    constexpr int kR = (32 * W + 1 + 63) / 64;
    uint32_t c[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int b = 64 * r + lane;
      c[r] = b < nb ? hist[b] : 0u;
    }
    int T = -1, hmin = -1;
    uint32_t below = 0, run = 0;
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const uint32_t incl = wave_scan_incl(c[r]) + run;
      const uint32_t excl = incl - c[r];
      const bool hit = 64 * r + lane < nb && excl < static_cast<uint32_t>(Ni) && incl >= static_cast<uint32_t>(Ni);
      const uint64_t hm = __ballot(hit);
      if (T < 0 && hm != 0) {
        const int l = __builtin_ctzll(hm);
        T = 64 * r + l;
        below = __builtin_amdgcn_readlane(excl, l);
      }
      const uint64_t nz = __ballot(64 * r + lane < nb && c[r] > 0);
      if (hmin < 0 && nz != 0) hmin = 64 * r + __builtin_ctzll(nz);
      run = __builtin_amdgcn_readlane(incl, 63);
    }
    if (T < 0) T = d;  // unreachable: the visible count is >= N_i
    if (hmin < 0) hmin = 0;
    const uint32_t rtie = static_cast<uint32_t>(Ni) - below;
    double z = 0.0;
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int b = 64 * r + lane;
      const uint32_t cc = b < T ? c[r] : (b == T ? rtie : 0u);
      if (cc != 0) z += static_cast<double>(cc) * static_cast<double>(wtab[b - hmin]);  // b >= h_min here
    }
    z = wave_sum_f64(z);
    if (lane == 63) {
      sh_T = T;
      sh_hmin = hmin;
      sh_quota = static_cast<int>(rtie);
      const float zf = static_cast<float>(z);
      sh_invz = zf > 0.0f ? 1.0f / zf : 0.0f;
    }
  }
  __syncthreads();
  const uint32_t T = static_cast<uint32_t>(sh_T);
  const int hmin = sh_hmin;
  const uint32_t quota = static_cast<uint32_t>(sh_quota);

  // the kept list in key order: thread t takes keys 16 t .. 16 t + 15 (their
  // distances read back from the list's space), counts its keys below T and
  // tied with T, packed strict | ties << 16 (each total <= 16384, so the
  // halves never carry into each other), and gets the counts of the keys
  // before its own from a wave scan and the wave totals; walking its keys in
  // order, a key below T, or one of the first `quota` ties, goes to slot
  // (strict keys before) + min(ties before, quota)
  uint32_t hv[kOneKPT];
  {
    const uint4* hp = reinterpret_cast<const uint4*>(hkey + tid * kOneKPT);
#pragma unroll
    for (int i = 0; i < kOneKPT / 8; ++i) {
      const uint4 x = hp[i];
      const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hv[8 * i + 2 * k] = xs[k] & 0xFFFFu;
        hv[8 * i + 2 * k + 1] = xs[k] >> 16;
      }
    }
  }
  uint32_t c = 0;
#pragma unroll
  for (int u = 0; u < kOneKPT; ++u) c += (hv[u] < T ? 1u : 0u) + (hv[u] == T ? 0x10000u : 0u);
  const uint32_t incl = wave_scan_incl(c);
  if (lane == 63) wtot[wid] = incl;
  __syncthreads();  // also: every thread has its distances out of the list's space
  uint32_t b = incl - c;
#pragma unroll
  for (int i = 0; i < kOneWaves / 4; ++i) {
    const uint4 x = reinterpret_cast<const uint4*>(wtot)[i];
    b += (4 * i < wid ? x.x : 0u) + (4 * i + 1 < wid ? x.y : 0u) + (4 * i + 2 < wid ? x.z : 0u) +
         (4 * i + 3 < wid ? x.w : 0u);
  }
  uint32_t sb = b & 0xFFFFu, tb = b >> 16;
#pragma unroll
  for (int u = 0; u < kOneKPT; ++u) {
    const uint32_t h = hv[u];
    const bool strict = h < T, tie = h == T;
    if (strict || (tie && tb < quota))
      list[sb + min(tb, quota)] = (static_cast<uint32_t>(tid * kOneKPT + u) << 9) | (h - hmin);
    sb += strict ? 1u : 0u;
    tb += tie ? 1u : 0u;
  }
  const int nl = Ni;
  __syncthreads();  // the list is complete

  // gather this part's columns of the kept V rows: ns lanes per row, 8
  // features each; R row groups.  Each pass takes R * kRows list entries and
  // row group g the kRows consecutive ones at g * kRows (read as 16-byte LDS
  // vectors), so all kRows row loads of a lane are issued together.
  const int R = kOneThreads / ns;
  const int g = tid / ns, li = tid - (tid / ns) * ns;
  const int fw = 8 * ns;  // columns per row group in the sums below
  float acc[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) acc[f] = 0.0f;
  constexpr int kEs = VF32 ? 4 : 2;  // bytes per V element
  const unsigned char* vbase = static_cast<const unsigned char*>(a.v) + bh * static_cast<int64_t>(a.kstride) * d * kEs;
  // bf16 rows: 16 in flight per lane group (at two parts per row, one pass
  // over N = 2048: 20.9 us per decode against 21.1 with 8)
  constexpr int kRows = (VF32 || !kVec) ? 4 : 16;
  const int c0 = 8 * (s0 + li);
  if (g < R) {
    if constexpr (kVec) {
      // 16-byte aligned rows (bf16: d % 8 == 0, so every slot is whole; fp32:
      // d % 4 == 0, so the slot's second half is whole or wholly past the row)
      // read through a buffer over the visible rows with 32-bit offsets
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned char*>(vbase), 0, kend * d * kEs, 0x00020000);
      const int rowb = d * kEs, cb = c0 * kEs;
      const bool hi_in = !VF32 || c0 + 4 < d;
      for (int base = 0; base < nl; base += kRows * R) {
        const int ef = base + g * kRows;
        uint32_t ent[kRows];
        const uint4* lp = reinterpret_cast<const uint4*>(list + min(ef, kOneMaxList - kRows));
#pragma unroll
        for (int i = 0; i < kRows / 4; ++i) {
          const uint4 x = lp[i];
          ent[4 * i] = x.x; ent[4 * i + 1] = x.y; ent[4 * i + 2] = x.z; ent[4 * i + 3] = x.w;
        }
        uint32_t raw[kRows][VF32 ? 8 : 4];
        float wr[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          const bool ok = ef + r < nl;
          const int jj = min(static_cast<int>(ent[r] >> 9), kend - 1);
          wr[r] = ok ? wtab[min(static_cast<int>(ent[r] & 0x1FFu), d)] : 0.0f;
          const int off = jj * rowb + cb;
          const uint4 u0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
          raw[r][0] = u0.x; raw[r][1] = u0.y; raw[r][2] = u0.z; raw[r][3] = u0.w;
          if constexpr (VF32) {
            const uint4 u1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, off + 16, 0, 0));
            raw[r][4] = hi_in ? u1.x : 0u; raw[r][5] = hi_in ? u1.y : 0u;
            raw[r][6] = hi_in ? u1.z : 0u; raw[r][7] = hi_in ? u1.w : 0u;
          }
        }
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          float x[8];
          if constexpr (VF32) {
#pragma unroll
            for (int f = 0; f < 8; ++f) x[f] = __builtin_bit_cast(float, raw[r][f]);
          } else {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
              x[2 * f] = __builtin_bit_cast(float, raw[r][f] << 16);
              x[2 * f + 1] = __builtin_bit_cast(float, raw[r][f] & 0xFFFF0000u);
            }
          }
#pragma unroll
          for (int f = 0; f < 8; ++f) acc[f] = fmaf(wr[r], x[f], acc[f]);
        }
      }
    } else {
      // unaligned rows: element loads, bounds-checked per column
      for (int base = 0; base < nl; base += kRows * R) {
        const int ef = base + g * kRows;
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          const bool ok = ef + r < nl;
          const uint32_t ent = list[min(ef + r, kOneMaxList - 1)];
          const int64_t jj = min(static_cast<int>(ent >> 9), kend - 1);
          const float wgt = ok ? wtab[min(static_cast<int>(ent & 0x1FFu), d)] : 0.0f;
          float x[8];
          if constexpr (VF32) {
            const float* row = reinterpret_cast<const float*>(vbase) + jj * d;
#pragma unroll
            for (int f = 0; f < 8; ++f) x[f] = c0 + f < d ? row[c0 + f] : 0.0f;
          } else {
            const uint16_t* row = reinterpret_cast<const uint16_t*>(vbase) + jj * d;
#pragma unroll
            for (int f = 0; f < 8; ++f)
              x[f] = __builtin_bit_cast(float, c0 + f < d ? static_cast<uint32_t>(row[c0 + f]) << 16 : 0u);
          }
#pragma unroll
          for (int f = 0; f < 8; ++f) acc[f] = fmaf(wgt, x[f], acc[f]);
        }
      }
    }
  }
  __syncthreads();  // every group is done with the list: its space takes the group sums
  if (g < R) {
#pragma unroll
    for (int f = 0; f < 8; ++f) red[g * fw + 8 * li + f] = acc[f];
  }
  __syncthreads();
  // sum the R group sums in a fixed order: chunk k adds groups k, k + K, ...,
  // then one thread per column adds the K chunk sums in order
  const int K = kOneThreads / fw;  // >= 4 (fw <= 256); R >= K
  {
    const int cl = tid % fw, k = tid / fw;
    if (k < K) {
      float sum = 0.0f;
      for (int gg = k; gg < R; gg += K) sum += red[gg * fw + cl];
      red2[k * fw + cl] = sum;
    }
  }
  __syncthreads();
  const float invz = sh_invz;
  float* orow = a.out + bhq * static_cast<int64_t>(d);
  const int cbase = 8 * s0;
  if (tid < fw && cbase + tid < d) {
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) sum += red2[k * fw + tid];
    orow[cbase + tid] = sum * invz;
  }
}

// Work split and workspace layout, from the shape alone.  keys_per_split is
// 256 times a power of two (at most 2048).  The per-(row, key) distance bins
// are kept when n_q <= W (n_q bytes per key against the 4W bytes of key
// words they replace in the gather; with more rows the key words, shared by
// the rows and served from L2, are cheaper), when every distance fits a byte
// (d <= 255: at d = 256 a key whose signs all differ from the row's has
// h = 256) and at most 1 GiB in all.
struct DecPlan {
  int splits, keys_per_split;
  bool bins;
  int64_t nkp;
  size_t off_hist, off_stats, off_part, off_bins, off_qbits, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

DecPlan plan_for(const had_decode_shape& s) {
  DecPlan p{};
  const int64_t rows = s.batch * s.heads * s.n_q;
  const int64_t nk = s.n_k;
  // aim at >= 1024 gather work-groups; at 4 x 32 rows against 16384 keys,
  // 1024 of them (2048-key splits) measured 28.4 us per decode, 2048 29.0 us
  // and 4096 41.4 us
  int64_t splits = (1024 + rows - 1) / rows;
  const int64_t max_by_keys = (nk + kDecMinKeysPerSplit - 1) / kDecMinKeysPerSplit;
  const int64_t min_by_keys = (nk + kDecMaxKeysPerSplit - 1) / kDecMaxKeysPerSplit;
  if (splits > max_by_keys) splits = max_by_keys;
  if (splits < min_by_keys) splits = min_by_keys;
  if (splits > kDecMaxSplits) splits = kDecMaxSplits;
  if (splits < 1) splits = 1;
  const int64_t want = (nk + splits - 1) / splits;
  int64_t per = kDecThreads;
  while (per < want && per < kDecMaxKeysPerSplit) per *= 2;
  splits = (nk + per - 1) / per;
  p.splits = static_cast<int>(splits);
  p.keys_per_split = static_cast<int>(per);
  p.nkp = splits * per;
  const size_t bins_bytes = static_cast<size_t>(rows) * static_cast<size_t>(p.nkp);
  p.bins = s.n_q <= words_per_row(s.dim) && s.dim <= 255 && bins_bytes <= (static_cast<size_t>(1) << 30);
  size_t off = 0;
  p.off_hist = off;
  off = align256(off + static_cast<size_t>(rows) * p.splits * (s.dim + 1) * sizeof(uint32_t));
  p.off_stats = off;
  off = align256(off + static_cast<size_t>(rows) * 4 * sizeof(int32_t));
  p.off_part = off;
  off = align256(off + static_cast<size_t>(rows) * p.splits * s.dim * sizeof(float));
  p.off_bins = off;
  if (p.bins) off = align256(off + bins_bytes);
  p.off_qbits = off;  // the new rows' sign words (had_decode_forward)
  off = align256(off + static_cast<size_t>(rows) * words_per_row(s.dim) * sizeof(uint32_t));
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

template <int W, bool kQF>
void launch_hist_q(const DecArgs& a, bool kvec, int64_t blocks, hipStream_t st) {
  if constexpr (W % 2 == 0) {
    if (kvec) {
      dec_hist_kernel<W, true, kQF><<<static_cast<unsigned>(blocks), kDecThreads, 0, st>>>(a);
      return;
    }
  }
  dec_hist_kernel<W, false, kQF><<<static_cast<unsigned>(blocks), kDecThreads, 0, st>>>(a);
}

template <int W>
void launch_hist(const DecArgs& a, bool kvec, int64_t blocks, hipStream_t st) {
  if (a.qf != nullptr) launch_hist_q<W, true>(a, kvec, blocks, st);
  else launch_hist_q<W, false>(a, kvec, blocks, st);
}

template <int W, bool kKVec, bool kBins>
void launch_gather_k(const DecArgs& a, bool vec, int64_t blocks, hipStream_t st) {
  const unsigned nb = static_cast<unsigned>(blocks);
  const size_t lds = gather_lds_bytes(a.keys_per_split);
  if (a.vf32) {
    if (vec) dec_gather_kernel<W, true, true, kKVec, kBins><<<nb, kDecThreads, lds, st>>>(a);
    else dec_gather_kernel<W, true, false, kKVec, kBins><<<nb, kDecThreads, lds, st>>>(a);
  } else {
    if (vec) dec_gather_kernel<W, false, true, kKVec, kBins><<<nb, kDecThreads, lds, st>>>(a);
    else dec_gather_kernel<W, false, false, kKVec, kBins><<<nb, kDecThreads, lds, st>>>(a);
  }
}

template <int W>
void launch_gather(const DecArgs& a, bool vec, bool kvec, int64_t blocks, hipStream_t st) {
  if (a.bins != nullptr) {
    launch_gather_k<W, false, true>(a, vec, blocks, st);
  } else if constexpr (W % 2 == 0) {
    if (kvec) launch_gather_k<W, true, false>(a, vec, blocks, st);
    else launch_gather_k<W, false, false>(a, vec, blocks, st);
  } else {
    launch_gather_k<W, false, false>(a, vec, blocks, st);
  }
}

// Compute units of the current device (cached per device; 256 if the runtime
// cannot say).
int device_cus() {
  static std::atomic<int> cache[64];  // 0: not known yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      return 256;
    }
    cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// Work-groups per (slice, row) on the single-launch path: double them (up to
// 4) while the pairs alone would leave CUs without a work-group and every part
// still gets at least one 8-column slot.  (At 128 pairs, 2 parts measured
// 23.5 us per decode and 4 parts 24.1 us: each part repeats the key scan.)
int one_fparts(int64_t rows, int d) {
  const int slots = (d + 7) / 8;
  const int cus = device_cus();
  int p = 1;
  while (p < 4 && rows * p < cus) {
    const int q = 2 * p;
    if ((q - 1) * ((slots + q - 1) / q) >= slots) break;
    p = q;
  }
  return p;
}

template <int W, bool VF32, bool kVec, bool kKVec>
void launch_one_q(const DecArgs& a, int64_t rows, hipStream_t st) {
  // work-group index: by slice (8 slices or more) or by pair, as in the kernel
  const unsigned nb = static_cast<unsigned>(a.bh_total >= 8 ? (a.bh_total + 7) / 8 * 8 * a.nq * a.fparts
                                                            : (rows + 7) / 8 * 8 * a.fparts);
  if (a.qf != nullptr)
    dec_one_kernel<W, VF32, kVec, kKVec, true><<<nb, kOneThreads, 0, st>>>(a);
  else
    dec_one_kernel<W, VF32, kVec, kKVec, false><<<nb, kOneThreads, 0, st>>>(a);
}

template <int W, bool VF32, bool kVec>
void launch_one_k(const DecArgs& a, bool kvec, int64_t rows, hipStream_t st) {
  if constexpr (W % 2 == 0) {
    if (kvec) {
      launch_one_q<W, VF32, kVec, true>(a, rows, st);
      return;
    }
  }
  launch_one_q<W, VF32, kVec, false>(a, rows, st);
}

template <int W>
void launch_one(const DecArgs& a, bool vec, bool kvec, int64_t rows, hipStream_t st) {
  if (a.vf32) {
    if (vec) launch_one_k<W, true, true>(a, kvec, rows, st);
    else launch_one_k<W, true, false>(a, kvec, rows, st);
  } else {
    if (vec) launch_one_k<W, false, true>(a, kvec, rows, st);
    else launch_one_k<W, false, false>(a, kvec, rows, st);
  }
}

}  // namespace
}  // namespace had

using namespace had;

extern "C" size_t had_decode_workspace_bytes(had_decode_shape s) {
  if (check_decode_shape(s) != HAD_OK) return 0;
  return plan_for(s).bytes;
}

namespace had {
namespace {

// had_decode (qbits given) and had_decode_forward (float32 rows qf, whose
// sign words the histogram launch builds into the workspace).
had_status decode_impl(const char* who, const uint32_t* qbits, const float* qf, const uint32_t* kbits,
                       const void* v, int v_dtype, had_decode_shape s, int64_t q_pos0,
                       int64_t topn, float scale, int causal, float* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  had_status st = check_decode_shape(s);
  if (st != HAD_OK) return st;
  const void* q = qf != nullptr ? static_cast<const void*>(qf) : static_cast<const void*>(qbits);
  if (q == nullptr || kbits == nullptr || v == nullptr || out == nullptr)
    return failf(HAD_ERR_INVALID_ARG, "%s: null queries, kbits, v or out", who);
  if (!aligned(q, 4) || !aligned(kbits, 4) || !aligned(v, 4) || !aligned(out, 4))
    return failf(HAD_ERR_INVALID_ARG, "%s: queries, kbits, v and out must be 4-byte aligned", who);
  if (!valid_dtype(v_dtype)) return failf(HAD_ERR_INVALID_ARG, "%s: unknown v_dtype", who);
  if (topn < 1) return failf(HAD_ERR_INVALID_ARG, "%s: topn must be >= 1", who);
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return failf(HAD_ERR_INVALID_ARG, "%s: scale must be finite and > 0", who);
  if (causal != 0 && causal != 1) return failf(HAD_ERR_INVALID_ARG, "%s: causal must be 0 or 1", who);
  if (q_pos0 < 0 || q_pos0 > HAD_MAX_DECODE_KEYS)
    return failf(HAD_ERR_INVALID_ARG, "%s: q_pos0 must be in [0, HAD_MAX_DECODE_KEYS]", who);
  const DecPlan p = plan_for(s);
  if (workspace == nullptr || !aligned(workspace, 256))
    return failf(HAD_ERR_INVALID_ARG, "%s: workspace must be non-null and 256-byte aligned", who);
  if (workspace_bytes < p.bytes)
    return failf(HAD_ERR_INVALID_ARG, "%s: workspace smaller than had_decode_workspace_bytes()", who);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  DecArgs a{};
  // the forward call builds the rows' words into the workspace
  a.qbits = qf != nullptr ? reinterpret_cast<const uint32_t*>(ws + p.off_qbits) : qbits;
  a.qf = qf;
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
  a.hist = reinterpret_cast<uint32_t*>(ws + p.off_hist);
  a.stats = reinterpret_cast<int32_t*>(ws + p.off_stats);
  a.part = reinterpret_cast<float*>(ws + p.off_part);
  a.bins = p.bins ? ws + p.off_bins : nullptr;
  a.nkp = p.nkp;
  a.splits = p.splits;
  a.keys_per_split = p.keys_per_split;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int64_t nqb = (s.n_q + kDecQBatch - 1) / kDecQBatch;
  const int64_t hist_blocks = a.bh_total * nqb * p.splits;
  const int64_t gather_blocks = a.bh_total * s.n_q * p.splits;
  const int64_t rows = a.bh_total * s.n_q;
  if (hist_blocks > 0x7FFFFFFF || gather_blocks > 0x7FFFFFFF || rows > 0x7FFFFFFF)
    return failf(HAD_ERR_UNSUPPORTED, "%s: grid too large", who);
  // key rows of W words load as 16-byte (W % 4 == 0) or 8-byte (W % 2 == 0)
  // vectors from an aligned base
  const bool kvec = aligned(kbits, a.W % 4 == 0 ? 16 : 8);
  // 16-byte row slices need 16-byte aligned rows
  const bool vec = aligned(v, 16) && (a.vf32 ? (a.d % 4 == 0) : (a.d % 8 == 0));
  // Few rows: fparts work-groups per (slice, row), one launch.  Each of its
  // work-groups scans the keys for one row, where the split histogram launch
  // reads a key once for up to 16 rows; at 16 new rows per slice (4 x 32
  // slices, 16384 keys) the single launch measured 174 us and the split
  // launches 186 us.
  if (rows <= kOneMaxPairs && s.n_q <= kOneMaxRows && s.n_k <= kOneMaxKeys && a.topn <= kOneMaxList) {
    a.fparts = one_fparts(rows, a.d);
    switch (a.W) {
      case 1: launch_one<1>(a, vec, kvec, rows, hs); break;
      case 2: launch_one<2>(a, vec, kvec, rows, hs); break;
      case 3: launch_one<3>(a, vec, kvec, rows, hs); break;
      case 4: launch_one<4>(a, vec, kvec, rows, hs); break;
      case 5: launch_one<5>(a, vec, kvec, rows, hs); break;
      case 6: launch_one<6>(a, vec, kvec, rows, hs); break;
      case 7: launch_one<7>(a, vec, kvec, rows, hs); break;
      default: launch_one<8>(a, vec, kvec, rows, hs); break;
    }
    return check_launch(who);
  }
  switch (a.W) {
    case 1: launch_hist<1>(a, kvec, hist_blocks, hs); break;
    case 2: launch_hist<2>(a, kvec, hist_blocks, hs); break;
    case 3: launch_hist<3>(a, kvec, hist_blocks, hs); break;
    case 4: launch_hist<4>(a, kvec, hist_blocks, hs); break;
    case 5: launch_hist<5>(a, kvec, hist_blocks, hs); break;
    case 6: launch_hist<6>(a, kvec, hist_blocks, hs); break;
    case 7: launch_hist<7>(a, kvec, hist_blocks, hs); break;
    default: launch_hist<8>(a, kvec, hist_blocks, hs); break;
  }
  if ((st = check_launch(who)) != HAD_OK) return st;
  switch (a.W) {
    case 1: launch_gather<1>(a, vec, kvec, gather_blocks, hs); break;
    case 2: launch_gather<2>(a, vec, kvec, gather_blocks, hs); break;
    case 3: launch_gather<3>(a, vec, kvec, gather_blocks, hs); break;
    case 4: launch_gather<4>(a, vec, kvec, gather_blocks, hs); break;
    case 5: launch_gather<5>(a, vec, kvec, gather_blocks, hs); break;
    case 6: launch_gather<6>(a, vec, kvec, gather_blocks, hs); break;
    case 7: launch_gather<7>(a, vec, kvec, gather_blocks, hs); break;
    default: launch_gather<8>(a, vec, kvec, gather_blocks, hs); break;
  }
  if ((st = check_launch(who)) != HAD_OK) return st;
  dec_reduce_kernel<<<static_cast<unsigned>(rows), (a.d + 63) / 64 * 64, 0, hs>>>(a);
  return check_launch(who);
}

}  // namespace
}  // namespace had

extern "C" had_status had_decode(const uint32_t* qbits, const uint32_t* kbits, const void* v,
                                 had_dtype v_dtype, had_decode_shape s, int64_t q_pos0,
                                 int64_t topn, float scale, int causal, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  if (qbits == nullptr) return fail(HAD_ERR_INVALID_ARG, "had_decode: null qbits");
  return decode_impl("had_decode", qbits, nullptr, kbits, v, enum_bits(v_dtype), s, q_pos0, topn, scale, causal, out,
                     workspace, workspace_bytes, stream);
}

extern "C" had_status had_decode_forward(const float* q, const uint32_t* kbits, const void* v,
                                         had_dtype v_dtype, had_decode_shape s, int64_t q_pos0,
                                         int64_t topn, float scale, int causal, float* out,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  if (q == nullptr) return fail(HAD_ERR_INVALID_ARG, "had_decode_forward: null q");
  return decode_impl("had_decode_forward", nullptr, q, kbits, v, enum_bits(v_dtype), s, q_pos0, topn, scale, causal,
                     out, workspace, workspace_bytes, stream);
}
