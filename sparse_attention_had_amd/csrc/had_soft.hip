// had_soft: the scaled-tanh (soft-binarized) forward of the HAD path.
//
// Method (Pith review of "Hamming Attention Distillation", section "What
// carries the argument"): the first training stages replace the sign of the
// standardized Q and K by a scaled tanh whose scale c decays, so that it
// approaches the sign smoothly; the referee's minor comment 1 notes that the
// form (Eqs. 13/15) is printed twice and never settled.  Read here as
// B_c(x) = tanh(x / (sigma * c)), c > 0, with the rest of the path unchanged:
// the logits are the real dot products s_ij = B_c(q_i) . B_c(k_j), every query
// row keeps its N_i = min(N, visible_i) largest logits (the lower key index
// first among equal ones, causal mask first), and the softmax of scale * s over
// the kept set weights the full-precision V rows.
//
// GPU design (gfx950), two launches:
//  1. transform: K -> B_c(K) in float32, rows padded with zeros to DP = 32,
//     64 or 128 features (one HBM pass each way).  The attention launch forms
//     B_c(Q) of its own 32 query rows while it stages them.
//  2. attention: a work-group is 8 waves (4 for n <= 256) and 32 query rows
//     of one (batch, head) slice, n <= 1024.  Wave w of W forms the 32 x 32
//     logit tiles of key tiles w, w + W, ... on the fp32 matrix cores
//     (v_mfma_f32_32x32x2f32, A = the key rows, the next tile's requested
//     before the current tile's products at d <= 64, B = the query rows staged
//     in LDS; lane L then holds query row L % 32 and 16 keys of each tile) and
//     keeps them in registers: at most 4 tiles of 16 values per lane.  The kept set is an exact radix select
//     over the composite (order-preserving bits of the float32 logit, then
//     the key index inverted), so exactly N_i keys are kept with no separate
//     tie rule: four levels of 8-bit digits of the logit's key and two of
//     5-bit digits of the index, each a per-row LDS histogram of the
//     elements still matching the prefix (ds_add_u32) and a scan that finds
//     the digit holding the N_i-th largest.  Then the row maximum, the
//     weights exp(scale * (s - max)) of the kept keys, their sum Z, and the
//     weighted V rows on the matrix cores, reduced over the waves in a fixed
//     order and divided by Z.  A row is resolved as soon as its quota takes a
//     whole bin, and the levels stop once every row is.  bf16 V (d a multiple
//     of 16): each wave stages its tile of 32 keys and up to 64 features (two
//     32-feature blocks per pass over the tiles) in LDS with 16-byte loads, in
//     the histogram area the select no longer needs (at d = 64 by asynchronous
//     global -> LDS copies into two buffers, the next tile's copies running
//     during the current tile's products), and reads the operand back
//     transposed (ds_read_b64_tr_b16); each float32 weight is split exactly into
//     three bf16 values, once per tile and pass, for v_mfma_f32_32x32x16_bf16.
//     fp32 V: the weights straight from the logit registers and V rows from L2
//     on the fp32 matrix cores.
// No floating-point atomics: results are identical run to run.
#include <algorithm>
#include <cmath>

#include "had_internal.h"

namespace had {
namespace {

// A work-group holds 32 query rows and every key: 8 waves of 4 key tiles for
// n <= 1024, or 4 waves of 2 key tiles for n <= 256 (no idle waves at short n).
template <int NW>
struct SoftCfg {
  static constexpr int kWaves = NW;
  static constexpr int kThreads = 64 * NW;
  static constexpr int kTiles = NW == 8 ? 4 : 2;        // key tiles per wave
  static constexpr int kScanLanes = 64 * NW / 32;       // lanes per row in the scans
};
constexpr int kSoftMaxSeq = 1024;                            // keys a work-group keeps in registers
constexpr int kBins = 256;                                   // histogram bins per row and level
// LDS histogram row stride (words): 16-byte rows for the scan's vector reads;
// 260 = 4 (mod 64) puts the 32 rows' copies of one bin on 16 banks.
constexpr int kHistStride = 260;

typedef float v16f __attribute__((ext_vector_type(16)));

// MFMA output register i of lane half `half`: the 32 x 32 tile's lane L holds
// column L % 32 and rows 8*(i/4) + 4*half + i%4.
__device__ inline int tile_row(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

// Unsigned key whose order is the float order (-0 is folded onto +0 first).
__device__ inline uint32_t order_key(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The float whose order key is k (k != 0).
__device__ inline float key_value(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

inline int soft_dp(int64_t d) { return d <= 32 ? 32 : (d <= 64 ? 64 : 128); }
inline size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// ---- 1. transform ----------------------------------------------------------
// K -> B_c(K) in float32, rows padded with zeros to DP features.  (The query
// rows are transformed by the attention launch itself, as it stages them.)
struct SoftTransformArgs {
  const float* x;
  float* xs;
  const float* sigma;  // device scalar or null (1)
  int64_t rows;        // B*H*n
  int d, dp, dp4_log2; // dp / 4 == 1 << dp4_log2
  int vec;             // d % 4 == 0 and x 16-byte aligned: float4 loads
  float c;
};

constexpr int kTfThreads = 256;

// 1 / (sigma c) in float32, at most FLT_MAX: a sigma of 0 (a constant tensor)
// or a subnormal c then still gives tanh(0) = 0 for x = 0 instead of 0 * inf.
__device__ inline float soft_mul(const float* sigma, float c) {
  const float sg = sigma != nullptr ? *sigma : 1.0f;
  return static_cast<float>(fmin(1.0 / (static_cast<double>(sg) * static_cast<double>(c)), 3.4028234663852886e38));
}

// Four soft features f .. f + 3 of row x (zeros past d).
__device__ inline float4 soft_four(const float* x, int f, int d, bool vec, float mul) {
  float4 y;
  if (vec && f + 4 <= d) {
    const float4 v = *reinterpret_cast<const float4*>(x + f);
    y = make_float4(tanhf(v.x * mul), tanhf(v.y * mul), tanhf(v.z * mul), tanhf(v.w * mul));
  } else {
    y.x = f < d ? tanhf(x[f] * mul) : 0.0f;
    y.y = f + 1 < d ? tanhf(x[f + 1] * mul) : 0.0f;
    y.z = f + 2 < d ? tanhf(x[f + 2] * mul) : 0.0f;
    y.w = f + 3 < d ? tanhf(x[f + 3] * mul) : 0.0f;
  }
  return y;
}

__global__ __launch_bounds__(kTfThreads) void soft_transform_kernel(SoftTransformArgs a) {
  const float mul = soft_mul(a.sigma, a.c);
  const int64_t groups = a.rows << a.dp4_log2;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kTfThreads;
  for (int64_t gi = static_cast<int64_t>(blockIdx.x) * kTfThreads + threadIdx.x; gi < groups; gi += stride) {
    const int64_t row = gi >> a.dp4_log2;
    const int f = 4 * static_cast<int>(gi & ((1 << a.dp4_log2) - 1));
    *reinterpret_cast<float4*>(a.xs + row * a.dp + f) = soft_four(a.x + row * a.d, f, a.d, a.vec != 0, mul);
  }
}

// Zero fill of the keep mask (a kernel, so that a captured graph holds no memset node).
__global__ __launch_bounds__(256) void soft_clear_kernel(uint8_t* p, int64_t bytes) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < bytes; i += stride) p[i] = 0;
}

// ---- 2. attention ----------------------------------------------------------
struct SoftArgs {
  const float* q;        // [BH, n, d] float32: the query rows, transformed while staged
  const float* sigma_q;  // device scalar or null (1)
  float c;
  int qvec;              // d % 4 == 0 and q 16-byte aligned
  const float* ks;       // [BH, n, DP] the soft key rows
  const void* v;    // [BH, n, d] float32 or bf16
  float* out;       // [BH, n, d]
  uint8_t* keep;    // mask mode: [bh_count, n, n], pre-cleared; 1 where kept
  int64_t bh_begin, bh_count;
  int n, d, topn;
  float scale;
  int causal;
  int vlds;         // bf16 V, d % 16 == 0, 16-byte aligned: V operands through LDS
};

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool VF32>
__device__ inline float load_v(const void* v, int64_t off) {
  if (VF32) return static_cast<const float*>(v)[off];
  const uint32_t b = static_cast<const uint16_t*>(v)[off];
  return __builtin_bit_cast(float, b << 16);
}

// One level of the radix select over the composite (order key of the logit,
// inverted key index): a per-row histogram of the digit of the elements that
// still match the prefix found so far, then the scan that finds the digit
// holding the row's remaining quota.  Levels 0-3 take the four bytes of the
// order key (highest first), levels 4 and 5 the two 5-bit digits of the key
// index, inverted so that lower indices come first among equal logits.  The
// key registers hold order keys, 0 for keys the row does not see: a visible key's
// top byte is never 0 (|s| <= d), so those sit below every visible one.  A row
// is resolved once its remaining quota takes the whole chosen bin: its
// threshold becomes the lowest composite of that bin.  All threads of the
// work-group call it; it returns (uniformly) whether every row is resolved.
template <int L, int NW>
__device__ __forceinline__ bool select_level(const uint32_t (&key)[SoftCfg<NW>::kTiles][16], uint32_t* hist, uint32_t* st_key,
                                             int* st_idx, int* st_need, int* st_done, int wid, int lane,
                                             int ntk) {
  using C = SoftCfg<NW>;
  const int half = lane >> 5, ql = lane & 31;
  const uint32_t kpre = st_key[ql];
  const int ipre = st_idx[ql];
  uint32_t* hrow = hist + ql * kHistStride;
#pragma unroll
  for (int u = 0; u < C::kTiles; ++u) {
    const int kt = wid + C::kWaves * u;
    if (kt < ntk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t k = key[u][r];
        if constexpr (L == 0) {
          atomicAdd(hrow + (k >> 24), 1u);
        } else if constexpr (L < 4) {
          if ((k >> (32 - 8 * L)) == kpre) atomicAdd(hrow + ((k >> (24 - 8 * L)) & 255u), 1u);
        } else if constexpr (L == 4) {
          if (k == kpre) atomicAdd(hrow + (31 - kt), 1u);  // key j = 32 kt + ...: j >> 5 == kt
        } else {
          if (k == kpre && kt == ipre) atomicAdd(hrow + (31 - tile_row(r, half)), 1u);
        }
      }
    }
  }
  __syncthreads();
  {
    // each wave scans 32 / W rows, 64 W / 32 lanes per row; lane g holds bins
    // kPer * g .. kPer * g + kPer - 1 of its row
    constexpr int kPer = (L < 4 ? kBins : 32) / C::kScanLanes;
    const int srow = (32 / C::kWaves) * wid + lane / C::kScanLanes, g = lane % C::kScanLanes;
    uint32_t* hb = hist + srow * kHistStride + kPer * g;
    const int nd = st_need[srow];
    uint32_t acc = 0, ct = 0;
    int tb = 0;
    bool mine = false;
    if constexpr (kPer % 4 == 0) {
      // 16-byte reads of groups of four bins; the lane holding the quota finds
      // its group from the group sums, re-reads that group (before the zeroing,
      // which LDS performs after it: one wave, in order) and finds the bin in it
      constexpr int kQ = kPer / 4;
      uint32_t gs[kQ];
      uint32_t sum = 0;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const uint4 x = *reinterpret_cast<const uint4*>(hb + 4 * q);
        gs[q] = (x.x + x.y) + (x.z + x.w);
        sum += gs[q];
      }
      uint32_t S = sum;  // bins of lanes g .. of the row, i.e. digits >= kPer * g
#pragma unroll
      for (int off = 1; off < C::kScanLanes; off <<= 1) {
        const uint32_t t = __shfl_down(S, off, C::kScanLanes);
        if (g + off < C::kScanLanes) S += t;
      }
      acc = S - sum;
      mine = nd > 0 && acc < static_cast<uint32_t>(nd) && static_cast<uint32_t>(nd) <= S;
      uint4 cg = {0u, 0u, 0u, 0u};
      int tq = 0;
      if (mine) {
        bool found = false;
#pragma unroll
        for (int q = kQ - 1; q >= 0; --q) {
          const bool hit = !found && acc + gs[q] >= static_cast<uint32_t>(nd);
          if (hit) {
            tq = q;
            found = true;
          }
          if (!found) acc += gs[q];
        }
        cg = *reinterpret_cast<const uint4*>(hb + 4 * tq);
      }
#pragma unroll
      for (int q = 0; q < kQ; ++q) *reinterpret_cast<uint4*>(hb + 4 * q) = uint4{0u, 0u, 0u, 0u};
      if (mine) {
        const uint32_t cc[4] = {cg.x, cg.y, cg.z, cg.w};
        bool found = false;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          const bool hit = !found && acc + cc[i] >= static_cast<uint32_t>(nd);
          if (hit) {
            tb = 4 * tq + i;
            ct = cc[i];
            found = true;
          }
          if (!found) acc += cc[i];
        }
      }
    } else {
      uint32_t c[kPer];
      uint32_t sum = 0;
#pragma unroll
      for (int b = 0; b < kPer; ++b) {
        c[b] = hb[b];
        sum += c[b];
      }
#pragma unroll
      for (int b = 0; b < kPer; ++b) hb[b] = 0u;
      uint32_t S = sum;
#pragma unroll
      for (int off = 1; off < C::kScanLanes; off <<= 1) {
        const uint32_t t = __shfl_down(S, off, C::kScanLanes);
        if (g + off < C::kScanLanes) S += t;
      }
      acc = S - sum;
      mine = nd > 0 && acc < static_cast<uint32_t>(nd) && static_cast<uint32_t>(nd) <= S;
      if (mine) {
        bool found = false;
#pragma unroll
        for (int b = kPer - 1; b >= 0; --b) {
          const bool hit = !found && acc + c[b] >= static_cast<uint32_t>(nd);
          if (hit) {
            tb = b;
            ct = c[b];
            found = true;
          }
          if (!found) acc += c[b];
        }
      }
    }
    if (mine) {
      const uint32_t digit = static_cast<uint32_t>(kPer * g + tb);
      const int rem = nd - static_cast<int>(acc);
      const bool whole = static_cast<uint32_t>(rem) == ct || L == 5;
      if constexpr (L < 4) {
        const uint32_t key = (L == 0 ? 0u : (st_key[srow] << 8)) | digit;
        st_key[srow] = whole ? key << (24 - 8 * L) : key;
        if (whole) st_idx[srow] = 0x7FFFFFFF;
      } else if constexpr (L == 4) {
        st_idx[srow] = whole ? 32 * (31 - static_cast<int>(digit)) + 31 : 31 - static_cast<int>(digit);
      } else {
        st_idx[srow] = 32 * st_idx[srow] + (31 - static_cast<int>(digit));
      }
      st_need[srow] = whole ? 0 : rem;
      if (whole) atomicAdd(st_done, 1);
    }
  }
  __syncthreads();
  return *st_done == 32;
}

template <int DP, bool VF32, bool MASK, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(4))) void soft_attn_kernel(SoftArgs a) {
  using C = SoftCfg<NW>;
  constexpr int HD = DP / 2;  // features of lane half h: h * HD .. h * HD + HD - 1
  constexpr int NFT = DP / 32;
  __shared__ __attribute__((aligned(16))) uint32_t hist[32 * kHistStride];  // per row, one level at a time; then the output partials
  __shared__ uint32_t st_key[32];        // logit key prefix, then the threshold key K*
  __shared__ int st_idx[32];             // index prefix, then the last kept index at K*
  __shared__ int st_need[32];            // kept keys still to place at the current level
  __shared__ int st_done;                // rows whose threshold is found
  __shared__ float red[C::kWaves][32];
  __shared__ uint32_t redk[C::kWaves][32];
  __shared__ __attribute__((aligned(16))) float qlds[32 * (DP + 4)];
  // d = 64 with 8 waves and bf16 V: the second buffer of the V tiles, then the second feature
  // block's partials (both blocks reduced after one barrier; the work-groups of this size are
  // held to two per CU by registers, not LDS)
  constexpr bool kPart1 = !MASK && !VF32 && NW == 8 && DP == 64;
  __shared__ __attribute__((aligned(16))) float part1[kPart1 ? NW * 1024 : 4];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, ql = lane & 31;
  const int n = a.n, d = a.d;
  const int nqt = (n + 31) / 32;
  const int64_t bh = a.bh_begin + blockIdx.x % a.bh_count;
  const int qt = nqt - 1 - static_cast<int>(blockIdx.x / a.bh_count);  // heaviest causal tiles first
  const int q0 = 32 * qt;
  const int i_row = q0 + ql;
  const bool rvalid = i_row < n;
  const int lim = !rvalid ? 0 : (a.causal ? i_row + 1 : n);  // row i sees keys j < lim
  const int kend = a.causal ? min(n, q0 + 32) : n;
  const int ntk = (kend + 31) / 32;  // key tiles some row of the block sees

  static_assert((32 * kHistStride) % 4 == 0, "histogram rows clear in 16-byte pieces");
  for (int e = tid; e < 8 * kHistStride; e += C::kThreads) reinterpret_cast<uint4*>(hist)[e] = uint4{0u, 0u, 0u, 0u};
  if (tid == 0) st_done = 0;
  // the block's 32 soft query rows B_c(q) (the B operand of every logit tile)
  {
    const float mulq = soft_mul(a.sigma_q, a.c);
    for (int e = tid; e < 8 * DP; e += C::kThreads) {
      const int row = e / (DP / 4), c4 = e % (DP / 4);
      const int i = min(q0 + row, n - 1);
      *reinterpret_cast<float4*>(qlds + row * (DP + 4) + 4 * c4) =
          soft_four(a.q + (bh * n + i) * d, 4 * c4, d, a.qvec != 0, mulq);
    }
  }
  __syncthreads();
  if (tid < 32) {
    // a row that keeps every key it sees (or a row past n) is resolved from
    // the start: threshold key 1 is below every visible key and above 0
    const int r = q0 + tid;
    const int vis = r >= n ? 0 : (a.causal ? r + 1 : n);
    const int need = min(a.topn, vis);
    const bool all = need == vis;
    st_need[tid] = all ? 0 : need;
    st_key[tid] = all ? 1u : 0u;
    st_idx[tid] = all ? 0x7FFFFFFF : 0;
    if (all) atomicAdd(&st_done, 1);
  }

  // ---- logits: s[u] = tile (key tile wid + 8u) x (the block's 32 rows)
  const float* qrow = qlds + ql * (DP + 4) + HD * half;  // B operand: the row's features t + HD * half
  v16f s[C::kTiles];
  if constexpr (DP <= 64) {
    // the next tile's key rows are requested before this tile's products
    // (at DP = 128 the second set of operands would not fit the register budget)
    float4 kx[HD / 4];
    auto kload = [&](int u) {
      const int kt = wid + C::kWaves * u;
      const int key = min(32 * kt + ql, n - 1);
      const float* kr = a.ks + (bh * n + key) * DP + HD * half;
#pragma unroll
      for (int t = 0; t < HD / 4; ++t) kx[t] = kt < ntk ? *reinterpret_cast<const float4*>(kr + 4 * t) : float4{};
    };
    kload(0);
#pragma unroll
    for (int u = 0; u < C::kTiles; ++u) {
      const int kt = wid + C::kWaves * u;
      float4 kc[HD / 4];
#pragma unroll
      for (int t = 0; t < HD / 4; ++t) kc[t] = kx[t];
      if (u + 1 < C::kTiles) kload(u + 1);
      v16f acc = {};
      if (kt < ntk) {
#pragma unroll
        for (int t = 0; t < HD; t += 4) {
          const float4 x = kc[t / 4];
          const float4 y = *reinterpret_cast<const float4*>(qrow + t);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.x, y.x, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.y, y.y, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.z, y.z, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.w, y.w, acc, 0, 0, 0);
        }
      }
      s[u] = acc;
    }
  } else {
#pragma unroll
    for (int u = 0; u < C::kTiles; ++u) {
      const int kt = wid + C::kWaves * u;
      v16f acc = {};
      if (kt < ntk) {
        const int key = min(32 * kt + ql, n - 1);
        const float* kr = a.ks + (bh * n + key) * DP + HD * half;
#pragma unroll
        for (int t = 0; t < HD; t += 4) {
          const float4 x = *reinterpret_cast<const float4*>(kr + t);
          const float4 y = *reinterpret_cast<const float4*>(qrow + t);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.x, y.x, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.y, y.y, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.z, y.z, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x.w, y.w, acc, 0, 0, 0);
        }
      }
      s[u] = acc;
      __builtin_amdgcn_sched_barrier(0);  // one tile's key rows in registers at a time
    }
  }
  // (no barrier here: the first level's barriers order the row state written above)

  // ---- exact top-N: radix select over (logit key, inverted index)
  // order keys of the logits, 0 for the keys this row does not see
  uint32_t key[C::kTiles][16];
#pragma unroll
  for (int u = 0; u < C::kTiles; ++u) {
    const int kt = wid + C::kWaves * u;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 32 * kt + tile_row(r, half);
      key[u][r] = (kt < ntk && j < lim) ? order_key(s[u][r]) : 0u;
    }
  }
  // the row maximum (the largest key, always kept): each wave's partial goes to LDS
  // here, and the first level's barrier publishes it
  {
    uint32_t mk = 0;
#pragma unroll
    for (int u = 0; u < C::kTiles; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) mk = max(mk, key[u][r]);
    mk = max(mk, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mk), 32)));
    if (!MASK && half == 0) redk[wid][ql] = mk;
  }
  if (!select_level<0, NW>(key, hist, st_key, st_idx, st_need, &st_done, wid, lane, ntk) &&
      !select_level<1, NW>(key, hist, st_key, st_idx, st_need, &st_done, wid, lane, ntk) &&
      !select_level<2, NW>(key, hist, st_key, st_idx, st_need, &st_done, wid, lane, ntk) &&
      !select_level<3, NW>(key, hist, st_key, st_idx, st_need, &st_done, wid, lane, ntk) &&
      !select_level<4, NW>(key, hist, st_key, st_idx, st_need, &st_done, wid, lane, ntk))
    select_level<5, NW>(key, hist, st_key, st_idx, st_need, &st_done, wid, lane, ntk);

  // key j of this row is kept iff visible and (key > K*, or key == K* and j <= j*)
  const uint32_t kst = st_key[ql];
  const int jst = st_idx[ql];

  if (MASK) {
    uint8_t* mrow = a.keep + ((bh - a.bh_begin) * n + (rvalid ? i_row : 0)) * static_cast<int64_t>(n);
#pragma unroll
    for (int u = 0; u < C::kTiles; ++u) {
      const int kt = wid + C::kWaves * u;
      if (kt < ntk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = 32 * kt + tile_row(r, half);
          const uint32_t k = key[u][r];
          if (k > kst || (k == kst && j <= jst)) mrow[j] = 1;
        }
      }
    }
    return;
  }

  // ---- weights and Z (the row maximum's partials are in redk since the first level)
  uint32_t rk = redk[0][ql];
#pragma unroll
  for (int w = 1; w < C::kWaves; ++w) rk = max(rk, redk[w][ql]);
  const float rmax = key_value(rk);
  const float c2 = a.scale * 1.4426950408889634f;
  const float off2 = rvalid ? rmax * c2 : 0.0f;
  float z = 0.0f;
#pragma unroll
  for (int u = 0; u < C::kTiles; ++u) {
    const int kt = wid + C::kWaves * u;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 32 * kt + tile_row(r, half);
      const uint32_t k = key[u][r];
      const bool keep = k > kst || (k == kst && j <= jst);
      const float p = keep ? exp2f(fmaf(key_value(k), c2, -off2)) : 0.0f;
      s[u][r] = p;
      z += p;
    }
  }
  z += __shfl_xor(z, 32);
  if (half == 0) red[wid][ql] = z;  // summed after the first barrier of the P V reduction

  // ---- out = P V / Z: passes over the key tiles, FC 32-feature blocks per pass (each
  // weight split once per pass), the waves' partials summed in LDS after each pass.  fp32
  // V takes one block per pass: it has no splits to share, and a second block's
  // accumulators and V rows would not fit the register budget.
  constexpr int FC = VF32 ? 1 : (NFT < 2 ? NFT : 2);
  static_assert(!kPart1 || FC == 2, "the one-barrier reduction takes two blocks");
  float* part = reinterpret_cast<float*>(hist);  // [waves][32 rows][32 features]
  static_assert(C::kWaves * 1024 <= 32 * kHistStride, "partials and V tiles fit the histogram area");
  // bf16 V tiles are staged in the histogram area as well (free once the select is
  // done): wave w's 32 keys x 32 FC features in the 4 KB its partials take later
  uint16_t* vst = reinterpret_cast<uint16_t*>(hist) + wid * 2048;
  const bool vlds = !VF32 && a.vlds;
  // bf16 V through LDS: lane L loads key 32 kt + L / 2, features 32 (fc + f) + 16 (L % 2)
  // .. + 15 of the wave's tile for each block f of the pass (two 16-byte loads per block,
  // rows clamped to n - 1, features past d read as zeros).  The loads are not issued a
  // tile ahead: holding them across the products spills registers (the other waves of
  // the SIMD cover their latency; at d = 64 the copies below need no registers).
  auto vload = [&](int fc, int u, uint4 (&pv)[2 * FC]) {
    const int kt = wid + C::kWaves * u;
    const int key = min(32 * kt + (lane >> 1), n - 1);
#pragma unroll
    for (int f = 0; f < FC; ++f) {
      const int fe = 32 * (fc + f) + 16 * (lane & 1);
      pv[2 * f] = uint4{0u, 0u, 0u, 0u};
      pv[2 * f + 1] = uint4{0u, 0u, 0u, 0u};
      if (fe < d && kt < ntk) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) + (bh * n + key) * d + fe);
        pv[2 * f] = src[0];
        pv[2 * f + 1] = src[1];
      }
    }
  };
  uint4 pv[2 * FC];
  float rz[1024 / C::kThreads];  // 1 / Z of the rows this thread writes
  // bf16 V with d = 64 and 8 waves: asynchronous global -> LDS copies (16 bytes per lane,
  // lane-ordered, no registers held), tile u in buffer u % 2 (the wave's 4 KB of the
  // histogram area, or of part1).  Copy i of block f holds keys 16 i .. 16 i + 15: lane L
  // brings key 16 i + L / 4, features 32 f + 8 (L % 4) .. + 7 (past d: feature 0, read
  // only by output columns that are dropped).  Tile u + 1 is requested right after tile
  // u's operands are read, so its copies run during tile u's products.
  auto vdma = [&](int uu) {
    const int kt2 = wid + C::kWaves * uu;
    if (kt2 < ntk) {
      uint16_t* db = (uu & 1) ? reinterpret_cast<uint16_t*>(part1) + wid * 2048 : vst;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int key = min(32 * kt2 + 16 * i + (lane >> 2), n - 1);
          const int fe0 = 32 * f + 8 * (lane & 3);
          const int fe = fe0 < d ? fe0 : 0;
          __builtin_amdgcn_global_load_lds(static_cast<const uint16_t*>(a.v) + (bh * n + key) * d + fe,
                                           (lds_void*)(db + f * 1024 + i * 512), 16, 0, 0);
        }
    }
  };
#pragma unroll
  for (int fc = 0; fc < NFT; fc += FC) {
    v16f o[FC];
#pragma unroll
    for (int f = 0; f < FC; ++f) o[f] = v16f{};
#pragma unroll
    for (int u = 0; u < C::kTiles; ++u) {
      const int kt = wid + C::kWaves * u;
      uint16_t* vb = vst;  // this tile's staged V
      if (vlds) {
        if constexpr (kPart1) {
          if (u == 0) vdma(0);
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: tile u has landed
          if (u & 1) vb = reinterpret_cast<uint16_t*>(part1) + wid * 2048;
        } else {
          vload(fc, u, pv);
          if (kt < ntk) {
#pragma unroll
            for (int f = 0; f < FC; ++f) {
              uint16_t* dst = vst + f * 1024 + (lane >> 1) * 32 + 16 * (lane & 1);
              *reinterpret_cast<uint4*>(dst) = pv[2 * f];
              *reinterpret_cast<uint4*>(dst + 8) = pv[2 * f + 1];
            }
          }
        }
        // one wave writes and reads its own tile: LDS keeps a wave's operations in
        // order, so only the compiler must not move the reads above the writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (kt < ntk) {
          // ds_read_b64_tr_b16: in each 16-lane group G, lane 4k + q gives the
          // address of (key S + k, features f0 + 4q .. f0 + 4q + 3) and lane j gets
          // (key S + k, feature f0 + j) for k = 0..3, with f0 = 16 (G % 2) and
          // S = 8 g + 4 (G / 2): keys 8 g + 4 half + k at feature 32 ft + L % 32,
          // the keys of this lane's weight registers 4g .. 4g + 3.
          // v_mfma_f32_32x32x16_bf16 sums 16 k-slots, slots 8 half .. 8 half + 7
          // from each lane: here the lane's registers 4 g0 .. 4 g0 + 7 (keys
          // 8 (g0 + i / 4) + 4 half + i % 4) in both operands.  Each float32 weight
          // is exactly hi + mid + lo, three bf16 values (the top 16 bits, those of
          // the remainder, the rest), so three bf16 products give P V with exact
          // partial products and float32 accumulation.
          const int G = lane >> 4, kk = (lane >> 2) & 3, qq = lane & 3;
          v8bf bv[2][FC];
#pragma unroll
          for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int f = 0; f < FC; ++f) {
              const uint16_t* tb = vb + f * 1024 + (16 * g + 4 * (G >> 1) + kk) * 32 + 16 * (G & 1) + 4 * qq;
              const v4s ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)tb);
              const v4s rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tb + 8 * 32));
              bv[g][f] = __builtin_bit_cast(v8bf, __builtin_shufflevector(ra, rb, 0, 1, 2, 3, 4, 5, 6, 7));
            }
          if constexpr (kPart1) {
            if (u + 1 < C::kTiles) vdma(u + 1);  // into the other buffer, during this tile's products
          }
#pragma unroll
          for (int g0 = 0; g0 < 4; g0 += 2) {
            uint32_t ph[8], pm[8], pl[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float x = s[u][4 * g0 + i];
              const uint32_t h = __builtin_bit_cast(uint32_t, x) & 0xFFFF0000u;
              const float r1 = x - __builtin_bit_cast(float, h);
              const uint32_t m = __builtin_bit_cast(uint32_t, r1) & 0xFFFF0000u;
              ph[i] = h;
              pm[i] = m;
              pl[i] = __builtin_bit_cast(uint32_t, r1 - __builtin_bit_cast(float, m));
            }
            u32x4 ah, am, al;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              ah[i] = __builtin_amdgcn_perm(ph[2 * i + 1], ph[2 * i], 0x07060302u);
              am[i] = __builtin_amdgcn_perm(pm[2 * i + 1], pm[2 * i], 0x07060302u);
              al[i] = __builtin_amdgcn_perm(pl[2 * i + 1], pl[2 * i], 0x07060302u);
            }
#pragma unroll
            for (int f = 0; f < FC; ++f) {
              o[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ah), bv[g0 / 2][f], o[f], 0, 0, 0);
              o[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, am), bv[g0 / 2][f], o[f], 0, 0, 0);
              o[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, al), bv[g0 / 2][f], o[f], 0, 0, 0);
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      } else if (kt < ntk) {
#pragma unroll
        for (int f = 0; f < FC; ++f) {
          const int feat = 32 * (fc + f) + ql;
          const bool fvalid = feat < d;
          float vv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = 32 * kt + tile_row(r, half);
            vv[r] = (j < n && fvalid) ? load_v<VF32>(a.v, (bh * n + j) * d + feat) : 0.0f;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) o[f] = __builtin_amdgcn_mfma_f32_32x32x2f32(s[u][r], vv[r], o[f], 0, 0, 0);
        }
      }
      // no instruction moves across tiles (the register budget holds one tile's operands)
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kPart1) {
      // one pass, blocks 0 (in the histogram area) and 1 (in part1) at once
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        part[wid * 1024 + tile_row(r, half) * 32 + ql] = o[0][r];
        part1[wid * 1024 + tile_row(r, half) * 32 + ql] = o[1][r];
      }
      __syncthreads();  // (it also publishes the waves' Z partials)
#pragma unroll
      for (int it = 0; it < 1024 / C::kThreads; ++it) {
        const int e = tid + it * C::kThreads;
        const int row = e >> 5, fo = e & 31;
        const int i = q0 + row;
        float Z = 0.0f;
#pragma unroll
        for (int w = 0; w < C::kWaves; ++w) Z += red[w][row];
        const float rzi = Z > 0.0f ? 1.0f / Z : 0.0f;
        if (i < n) {
          float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
          for (int w = 0; w < C::kWaves; ++w) {
            v0 += part[1024 * w + e];
            v1 += part1[1024 * w + e];
          }
          if (fo < d) a.out[(bh * n + i) * d + fo] = v0 * rzi;
          if (32 + fo < d) a.out[(bh * n + i) * d + 32 + fo] = v1 * rzi;
        }
      }
    } else {
#pragma unroll
    for (int f = 0; f < FC; ++f) {
      const int ft = fc + f;
      // a wave's partials take the LDS its own V tiles took, so only a later block
      // waits for the previous block's partials to be consumed
      if (f > 0) __syncthreads();
#pragma unroll
      for (int r = 0; r < 16; ++r) part[wid * 1024 + tile_row(r, half) * 32 + ql] = o[f][r];
      __syncthreads();  // (before the first block it also publishes the waves' Z partials)
#pragma unroll
      for (int it = 0; it < 1024 / C::kThreads; ++it) {
        const int e = tid + it * C::kThreads;
        const int row = e >> 5, fo = e & 31;
        const int i = q0 + row, fe = 32 * ft + fo;
        if (ft == 0) {  // this thread's rows are the same in every block
          float Z = 0.0f;
#pragma unroll
          for (int w = 0; w < C::kWaves; ++w) Z += red[w][row];
          rz[it] = Z > 0.0f ? 1.0f / Z : 0.0f;
        }
        if (i < n && fe < d) {
          float val = 0.0f;
#pragma unroll
          for (int w = 0; w < C::kWaves; ++w) val += part[1024 * w + e];
          a.out[(bh * n + i) * d + fe] = val * rz[it];
        }
      }
    }
    }
    if (fc + FC < NFT) __syncthreads();  // the partials are read before the next pass stages V over them
  }
}

template <int DP, bool MASK, int NW>
had_status launch_soft_attn(const SoftArgs& a, had_dtype vdt, hipStream_t st) {
  const int nqt = (a.n + 31) / 32;
  const dim3 grid(static_cast<unsigned>(a.bh_count * nqt));
  if (MASK || vdt == HAD_F32)
    hipLaunchKernelGGL((soft_attn_kernel<DP, true, MASK, NW>), grid, dim3(64 * NW), 0, st, a);
  else
    hipLaunchKernelGGL((soft_attn_kernel<DP, false, MASK, NW>), grid, dim3(64 * NW), 0, st, a);
  return check_launch("soft_attn_kernel");
}

template <int DP, bool MASK>
had_status launch_soft_attn(const SoftArgs& a, had_dtype vdt, hipStream_t st) {
  return a.n <= 256 ? launch_soft_attn<DP, MASK, 4>(a, vdt, st) : launch_soft_attn<DP, MASK, 8>(a, vdt, st);
}

template <bool MASK>
had_status launch_soft_attn_dp(const SoftArgs& a, int dp, had_dtype vdt, hipStream_t st) {
  if (dp == 32) return launch_soft_attn<32, MASK>(a, vdt, st);
  if (dp == 64) return launch_soft_attn<64, MASK>(a, vdt, st);
  return launch_soft_attn<128, MASK>(a, vdt, st);
}

had_status check_soft(const float* q, const float* k, const had_shape& s, int64_t topn, float c,
                      int causal, const float* sigma_q, const float* sigma_k, void* workspace,
                      size_t workspace_bytes, const char* fn) {
  had_status st = check_shape(s);
  if (st != HAD_OK) return st;
  if (s.dim > 128) return failf(HAD_ERR_UNSUPPORTED, "%s: dim above 128", fn);
  if (s.seq > HAD_SOFT_MAX_SEQ) return failf(HAD_ERR_UNSUPPORTED, "%s: seq above HAD_SOFT_MAX_SEQ (1024)", fn);
  if (q == nullptr || k == nullptr) return failf(HAD_ERR_INVALID_ARG, "%s: null q or k", fn);
  if (!aligned(q, 4) || !aligned(k, 4)) return failf(HAD_ERR_INVALID_ARG, "%s: q and k must be 4-byte aligned", fn);
  if ((sigma_q != nullptr && !aligned(sigma_q, 4)) || (sigma_k != nullptr && !aligned(sigma_k, 4)))
    return failf(HAD_ERR_INVALID_ARG, "%s: sigma pointers must be 4-byte aligned", fn);
  if (topn < 1) return failf(HAD_ERR_INVALID_ARG, "%s: topn must be >= 1", fn);
  if (!std::isfinite(c) || !(c > 0.0f)) return failf(HAD_ERR_INVALID_ARG, "%s: c must be finite and > 0", fn);
  if (causal != 0 && causal != 1) return failf(HAD_ERR_INVALID_ARG, "%s: causal must be 0 or 1", fn);
  if (workspace == nullptr || !aligned(workspace, 256))
    return failf(HAD_ERR_INVALID_ARG, "%s: workspace must be non-null and 256-byte aligned", fn);
  if (workspace_bytes < had_soft_workspace_bytes(s))
    return failf(HAD_ERR_INVALID_ARG, "%s: workspace smaller than had_soft_workspace_bytes()", fn);
  return HAD_OK;
}

// Launch 1 (the soft key rows) into the workspace; fills the input fields of a.
had_status soft_transform(const float* q, const float* k, const had_shape& s, float c, const float* sigma_q,
                          const float* sigma_k, void* workspace, SoftArgs& a, hipStream_t st) {
  const int dp = soft_dp(s.dim);
  const int64_t rows = s.batch * s.heads * s.seq;
  float* ks = static_cast<float*>(workspace);
  SoftTransformArgs t{};
  t.x = k;
  t.xs = ks;
  t.sigma = sigma_k;
  t.rows = rows;
  t.d = static_cast<int>(s.dim);
  t.dp = dp;
  t.dp4_log2 = dp == 32 ? 3 : (dp == 64 ? 4 : 5);
  t.vec = s.dim % 4 == 0 && aligned(k, 16);
  t.c = c;
  const int64_t groups = rows * (dp / 4);
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>((groups + kTfThreads - 1) / kTfThreads, 8192)));
  hipLaunchKernelGGL(soft_transform_kernel, grid, dim3(kTfThreads), 0, st, t);
  had_status r = check_launch("soft_transform_kernel");
  if (r != HAD_OK) return r;
  a.q = q;
  a.sigma_q = sigma_q;
  a.c = c;
  a.qvec = s.dim % 4 == 0 && aligned(q, 16);
  a.ks = ks;
  a.n = static_cast<int>(s.seq);
  a.d = static_cast<int>(s.dim);
  return HAD_OK;
}

}  // namespace
}  // namespace had

using namespace had;

extern "C" size_t had_soft_workspace_bytes(had_shape s) {
  if (check_shape(s) != HAD_OK || s.dim > 128 || s.seq > HAD_SOFT_MAX_SEQ) return 0;
  const size_t rows = static_cast<size_t>(s.batch * s.heads * s.seq);
  return align256(rows * soft_dp(s.dim) * sizeof(float));
}

extern "C" had_status had_soft_forward(const float* q, const float* k, const void* v, had_dtype v_dtype,
                                       had_shape s, int64_t topn, float scale, float c, int causal,
                                       const float* sigma_q, const float* sigma_k, float* out,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  had_status st = check_soft(q, k, s, topn, c, causal, sigma_q, sigma_k, workspace, workspace_bytes,
                             "had_soft_forward");
  if (st != HAD_OK) return st;
  if (v == nullptr || out == nullptr) return fail(HAD_ERR_INVALID_ARG, "had_soft_forward: null v or out");
  if (!aligned(v, 4) || !aligned(out, 4))
    return fail(HAD_ERR_INVALID_ARG, "had_soft_forward: v and out must be 4-byte aligned");
  const int vdt = enum_bits(v_dtype);
  if (!valid_dtype(vdt)) return fail(HAD_ERR_INVALID_ARG, "had_soft_forward: unknown v_dtype");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(HAD_ERR_INVALID_ARG, "had_soft_forward: scale must be finite and > 0");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  SoftArgs a{};
  if ((st = soft_transform(q, k, s, c, sigma_q, sigma_k, workspace, a, hs)) != HAD_OK) return st;
  a.v = v;
  a.out = out;
  a.vlds = vdt == HAD_BF16 && s.dim % 16 == 0 && aligned(v, 16);
  a.bh_begin = 0;
  a.bh_count = s.batch * s.heads;
  a.topn = static_cast<int>(topn > s.seq ? s.seq : topn);
  a.scale = scale;
  a.causal = causal;
  return launch_soft_attn_dp<false>(a, soft_dp(s.dim), static_cast<had_dtype>(vdt), hs);
}

extern "C" had_status had_soft_select(const float* q, const float* k, had_shape s, int64_t topn, float c,
                                      int causal, const float* sigma_q, const float* sigma_k,
                                      int64_t bh_begin, int64_t bh_count, uint8_t* keep, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  clear_error();
  had_status st = check_soft(q, k, s, topn, c, causal, sigma_q, sigma_k, workspace, workspace_bytes,
                             "had_soft_select");
  if (st != HAD_OK) return st;
  if (keep == nullptr) return fail(HAD_ERR_INVALID_ARG, "had_soft_select: null keep");
  const int64_t bht = s.batch * s.heads;
  if (bh_begin < 0 || bh_count < 1 || bh_begin + bh_count > bht)
    return fail(HAD_ERR_INVALID_ARG, "had_soft_select: slice range outside [0, B*H)");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int64_t keep_bytes = bh_count * s.seq * s.seq;
  hipLaunchKernelGGL(soft_clear_kernel, dim3(static_cast<unsigned>(std::min<int64_t>((keep_bytes + 255) / 256, 4096))),
                     dim3(256), 0, hs, keep, keep_bytes);
  if ((st = check_launch("soft_clear_kernel")) != HAD_OK) return st;
  SoftArgs a{};
  if ((st = soft_transform(q, k, s, c, sigma_q, sigma_k, workspace, a, hs)) != HAD_OK) return st;
  a.keep = keep;
  a.bh_begin = bh_begin;
  a.bh_count = bh_count;
  a.topn = static_cast<int>(topn > s.seq ? s.seq : topn);
  a.scale = 1.0f;
  a.causal = causal;
  return launch_soft_attn_dp<true>(a, soft_dp(s.dim), HAD_F32, hs);
}
