// had_backward: straight-through backward of the HAD attention path.
//
// Method (Pith review of "Hamming Attention Distillation", section "What
// carries the argument"): training runs a four-stage annealing schedule whose
// later stages finish the binarization with a straight-through estimator, so
// the forward pass is the inference path (sign-binarized Q and K, integer
// logits s = d - 2h, top-N per row with lower key index first among equal
// logits, softmax over the kept set, weighted sum of full-precision V) and
// the backward pass treats sign() as the identity on the standardized input.
// With the kept sets held fixed, for row i and p_ij = softmax over its kept
// set of scale * s_ij:
//
//   dP_ij = dout_i . V_j,   D_i = dout_i . out_i,   dS_ij = scale p_ij (dP_ij - D_i),
//   dV_j  = sum_i p_ij dout_i,
//   dQ_i  = (sum_j dS_ij Bk_j) / sigma_Q,   dK_j = (sum_i dS_ij Bq_i) / sigma_K.
//
// GPU design (gfx950), three launches:
//  1. Row statistics: the attention kernel's histogram pass in a statistics
//     mode writes per row the threshold bin T, h_min, Z and the index c of
//     the last kept key at the threshold.  Key j is then kept by row i iff it
//     is visible and h_ij < T_i, or h_ij == T_i and j <= c_i: a per-row test
//     that needs no running tie count, so the key-major launch can apply it.
//  2. dQ, query-major: a work-group is 4 waves x 32 query rows of one (batch,
//     head) slice; per tile of 32 consecutive keys (key words and V staged in
//     LDS), each wave forms the 32 x 32 tile of h by XOR + popcount (lane L
//     holds query L % 32 and 16 keys), the weights, dP on the fp32 matrix
//     cores (v_mfma_f32_32x32x2f32, A = the V tile, B = the row's dout held
//     in registers), dS, and accumulates dS * Bk on the matrix cores (A = the
//     +-1 key bits, B = dS straight from the tile registers).  It also writes
//     D_i = dout_i . out_i for launch 3.
//  3. dK and dV, key-major: a work-group is 4 waves x 32 keys; per tile of 32
//     query rows (their sign words, dout rows, statistics and D staged in
//     LDS) each wave forms h, the weights and dP (A = the dout tile, B = the
//     key's V row in registers), dS, and accumulates P^T dout and dS^T Bq.
// With fp32 V everything is float32 on the matrix cores (their fp32
// products round like the vector ALU's).  With bf16 V the products run on
// the bf16 matrix cores with the float32 operands split into three bf16
// terms (see the bf16 kernels below).  No floating-point atomics,
// so results are identical run to run.  Masked elements take weight 0.
#include <cmath>

#include "had_internal.h"

namespace had {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdRows = 32 * kBwdWaves;  // query rows (dQ) or keys (dK, dV) per work-group

struct BwdArgs {
  const uint32_t* qbits;  // [BH, n, W]
  const uint32_t* kbits;  // [BH, n, W]
  const void* v;          // [BH, n, d] float32 or bf16
  const float* out;       // [BH, n, d] the forward output
  const float* dout;      // [BH, n, d]
  const float* sigma_q;   // device scalar or null (1)
  const float* sigma_k;
  float* dq;              // [BH, n, d]
  float* dk;
  float* dv;
  const int32_t* stats;   // [BH, n, 4]: T, last kept tie, h_min, Z bits
  float* dsum;            // [BH, n]: D_i
  int64_t bh_total;
  int n, d;
  float scale;
  int causal;
};

typedef float v16f __attribute__((ext_vector_type(16)));

// MFMA row (key or query) of output register i in lane half `half`: the
// 32 x 32 tile's lane L holds column L % 32 and rows 8*(i/4) + 4*half + i%4.
__device__ inline int tile_row(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

__device__ inline float load_v(const void* v, int64_t off, bool vf32) {
  if (vf32) return static_cast<const float*>(v)[off];
  const uint32_t b = static_cast<const uint16_t*>(v)[off];
  return __builtin_bit_cast(float, b << 16);
}

// ---- 2. dQ (query-major) -------------------------------------------------
// Tiles of 32 keys are staged double-buffered: each thread requests its share
// of tile t + 1 (key words, V values) into registers before computing tile
// t, and writes it into the other LDS buffer afterwards, so the global loads
// run under the matrix-core work and one barrier per tile suffices.
template <int W, bool VF32>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(BwdArgs a) {
  constexpr int DP = 32 * W;   // padded features
  constexpr int VS = DP + 1;   // LDS row stride of the V tile (no bank conflicts)
  constexpr int kVPT = DP / 8; // V values per thread per tile (32 * DP / 256)
  __shared__ float vt[2][32 * VS];
  __shared__ uint32_t kw[2][32 * W];
  __shared__ float wtab[DP + 1];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, ql = lane & 31;
  const int n = a.n, d = a.d;
  const int ntq = (n + kBwdRows - 1) / kBwdRows;
  const int64_t bh = blockIdx.x % a.bh_total;
  const int qt = ntq - 1 - static_cast<int>(blockIdx.x / a.bh_total);  // heaviest causal tiles first
  const int q0 = qt * kBwdRows;
  const int i_row = q0 + 32 * wid + ql;
  const bool qvalid = i_row < n;
  const int lim = !qvalid ? 0 : (a.causal ? i_row + 1 : n);
  const int kend = a.causal ? min(n, q0 + kBwdRows) : n;
  const int ntiles = (kend + 31) / 32;
  const int wq0 = q0 + 32 * wid;
  const int wlim = wq0 >= n ? 0 : (a.causal ? min(n, wq0 + 32) : n);
  const int wtiles = (wlim + 31) / 32;  // tiles with keys this wave sees

  for (int t = tid; t <= d; t += kBwdThreads) wtab[t] = expf(-2.0f * a.scale * static_cast<float>(t));

  const int64_t row = bh * n + (qvalid ? i_row : 0);
  int T = 0, cut = -1, hmin = 0;
  float invZ = 0.0f;
  uint32_t qw[W];
  float dr[16 * W];  // dout[i_row][2s + half], s < 16W (the B operand of dP)
  float D = 0.0f;
  {
    const int4 st = *reinterpret_cast<const int4*>(a.stats + row * 4);
    T = st.x;
    cut = st.y;
    hmin = st.z;
    const float Z = __builtin_bit_cast(float, st.w);
    invZ = (qvalid && Z > 0.0f) ? 1.0f / Z : 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) qw[w] = a.qbits[row * W + w];
    const float* drow = a.dout + row * d;
    const float* orow = a.out + row * d;
    float part = 0.0f;
#pragma unroll
    for (int s = 0; s < 16 * W; ++s) {
      const int f = 2 * s + half;
      dr[s] = (qvalid && f < d) ? drow[f] : 0.0f;
      part = fmaf(dr[s], (qvalid && f < d) ? orow[f] : 0.0f, part);
    }
    D = part + __shfl_xor(part, 32, 64);  // both halves of the row
  }
  if (qvalid && half == 0) a.dsum[row] = D;

  v16f acc[W];
#pragma unroll
  for (int t = 0; t < W; ++t) acc[t] = v16f{};

  const uint32_t* kbase = a.kbits + bh * static_cast<int64_t>(n) * W;
  const int64_t vbase = bh * static_cast<int64_t>(n) * d;
  // Every thread loads from a valid (clamped) address unconditionally and
  // zeroes out-of-range values when it writes them, so all its loads are in
  // flight together.
  uint32_t pk = 0;
  uint32_t pv[kVPT];  // raw V values (fp32 bits or a bf16 in the low half)
  int staged_k0 = 0;  // first key of the tile in pk, pv
  auto prefetch = [&](int tile) {
    const int k0 = 32 * tile;
    staged_k0 = k0;
    pk = kbase[static_cast<int64_t>(min(k0 + min(tid, 32 * W - 1) / W, n - 1)) * W + tid % W];
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      const int e = tid + j * kBwdThreads;
      const int r = e / DP, f = e - r * DP;
      const int64_t off = vbase + static_cast<int64_t>(min(k0 + r, n - 1)) * d + min(f, d - 1);
      if constexpr (VF32)
        pv[j] = __builtin_bit_cast(uint32_t, static_cast<const float*>(a.v)[off]);
      else
        pv[j] = static_cast<const uint16_t*>(a.v)[off];
    }
  };
  auto commit = [&](int buf) {
    if (tid < 32 * W) kw[buf][tid] = pk;
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      const int e = tid + j * kBwdThreads;
      const int r = e / DP, f = e - r * DP;
      const bool in = staged_k0 + r < n && f < d;
      const float x = VF32 ? __builtin_bit_cast(float, pv[j]) : __builtin_bit_cast(float, pv[j] << 16);
      vt[buf][r * VS + f] = in ? x : 0.0f;
    }
  };
  prefetch(0);
  commit(0);
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    const int k0 = 32 * tile;
    if (tile + 1 < ntiles) prefetch(tile + 1);
    if (tile < wtiles) {
      const float* vtb = vt[buf];
      const uint32_t* kwb = kw[buf];
      // the 16 keys' words (also the +-1 operand of dS Bk below), their
      // distances and weights, branch-free so that the LDS reads issue together
      uint32_t kwv[16][W];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int w = 0; w < W; ++w) kwv[i][w] = kwb[tile_row(i, half) * W + w];
      }
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + tile_row(i, half);
        int h = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) h += __builtin_popcount(qw[w] ^ kwv[i][w]);
        const bool keep = (key < lim) & ((h < T) | ((h == T) & (key <= cut)));
        const float wt = wtab[min(max(h - hmin, 0), d)];
        p[i] = keep ? wt * invZ : 0.0f;
      }
      // dP tile: rows = keys, columns = query rows; the A operands of 8
      // products are read while the previous 8 run
      v16f dp = v16f{};
      constexpr int kS = 16 * W;
      float va[2][8];
#pragma unroll
      for (int k = 0; k < 8; ++k) va[0][k] = vtb[ql * VS + 2 * k + half];
#pragma unroll
      for (int c = 0; c < kS / 8; ++c) {
        if (c + 1 < kS / 8) {
#pragma unroll
          for (int k = 0; k < 8; ++k) va[(c + 1) & 1][k] = vtb[ql * VS + 2 * (8 * (c + 1) + k) + half];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
          dp = __builtin_amdgcn_mfma_f32_32x32x2f32(va[c & 1][k], dr[8 * c + k], dp, 0, 0, 0);
      }
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = a.scale * p[i] * (dp[i] - D);
      // dQ^T += Bk^T dS: A = +-1 of feature 32t + ql of key tile_row(i, half);
      // the W feature tiles' chains interleaved
#pragma unroll
      for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int t = 0; t < W; ++t) {
          const float b = ((kwv[i][t] >> ql) & 1u) ? -1.0f : 1.0f;
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(b, ds[i], acc[t], 0, 0, 0);
        }
      }
    }
    if (tile + 1 < ntiles) commit(buf ^ 1);
    __syncthreads();
  }
  if (!qvalid) return;
  const float g = a.sigma_q != nullptr ? 1.0f / *a.sigma_q : 1.0f;
  float* drow = a.dq + row * d;
#pragma unroll
  for (int t = 0; t < W; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int f = 32 * t + tile_row(i, half);
      if (f < d) drow[f] = acc[t][i] * g;
    }
  }
}

// ---- bf16 V: the products on the bf16 matrix cores ------------------------
// Every float32 x is exactly hi + mid + lo with three bf16 values (hi = the
// top 16 bits of x, mid the top 16 bits of the remainder, lo the rest, which
// has at most 8 significant bits).  A product with an operand that is exact
// in bf16 (the +-1 sign bits, bf16 V) is then three bf16 products with
// exact partial products and float32 accumulation; a product of two split
// float32 operands keeps six of the nine partial products (each dropped one
// is below 2^-21 of the product: |mid| < 2^-7 |x| and |lo| < 2^-14 |x|).
// v_mfma_f32_32x32x16_bf16 sums over 16 k-slots, slot s of lane half h in A
// and in B; the kernels give the slot (h, s) the same index on both sides:
// a feature 16 c + 8 h + s for the products over features, and for the
// products over the 32 keys (dQ) or query rows (dK, dV) of a tile the
// element 8 cc + s of the lane's own 32 x 32 tile registers (row
// tile_row(8 cc + s, h)), so dS and P feed the next products as they are.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Eight float32 values as three bf16 operand vectors (element s = x[s]);
// the top halves of two words are joined by one byte permute.
__device__ inline void split8(const float* x, v8bf* o) {
  u32x4 ph, pm, pl;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float xa = x[2 * k], xb = x[2 * k + 1];
    const uint32_t ua = __builtin_bit_cast(uint32_t, xa), ub = __builtin_bit_cast(uint32_t, xb);
    const float ra = xa - __builtin_bit_cast(float, ua & 0xFFFF0000u);
    const float rb = xb - __builtin_bit_cast(float, ub & 0xFFFF0000u);
    const uint32_t ura = __builtin_bit_cast(uint32_t, ra), urb = __builtin_bit_cast(uint32_t, rb);
    const float la = ra - __builtin_bit_cast(float, ura & 0xFFFF0000u);
    const float lb = rb - __builtin_bit_cast(float, urb & 0xFFFF0000u);
    ph[k] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);
    pm[k] = __builtin_amdgcn_perm(urb, ura, 0x07060302u);
    pl[k] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, lb), __builtin_bit_cast(uint32_t, la), 0x07060302u);
  }
  o[0] = __builtin_bit_cast(v8bf, ph);
  o[1] = __builtin_bit_cast(v8bf, pm);
  o[2] = __builtin_bit_cast(v8bf, pl);
}

// The +-1 operand: element s = -1 if bit `bit` of w[s] is set, else +1.
__device__ inline v8bf sign_operand(const uint32_t* w, int bit) {
  const int sh = 31 - bit;
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t s0 = (w[2 * k] << sh) >> 16;  // bit 15 = the sign of element 2k
    const uint32_t s1 = w[2 * k + 1] << sh;      // bit 31 = the sign of element 2k + 1
    o[k] = (s0 & 0x8000u) | (s1 & 0x80000000u) | 0x3F803F80u;
  }
  return __builtin_bit_cast(v8bf, o);
}

#define MFMA_BF16(a, b, c) __builtin_amdgcn_mfma_f32_32x32x16_bf16((a), (b), (c), 0, 0, 0)

// dQ, query-major, bf16 V.  As bwd_dq_kernel; the V tile is staged
// as bf16 rows, dout of the wave's rows is split once into bf16 operands,
// dP takes 3 products per 16 features and dQ^T += Bk^T dS 3 per 16 keys.
template <int W>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_bf_kernel(BwdArgs a) {
  static_assert(W <= 4, "d <= 128");
  constexpr int DP = 32 * W;
  constexpr int NC = DP / 16;   // 16-feature steps of dP
  constexpr int VSB = DP + 8;   // LDS row stride of the V tile, bf16 elements (16-byte rows, odd multiple)
  constexpr int kVPT = DP / 8;  // V values per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][32 * VSB];
  __shared__ uint32_t kw[2][32 * W];
  __shared__ float wtab[DP + 1];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, ql = lane & 31;
  const int n = a.n, d = a.d;
  const int ntq = (n + kBwdRows - 1) / kBwdRows;
  const int64_t bh = blockIdx.x % a.bh_total;
  const int qt = ntq - 1 - static_cast<int>(blockIdx.x / a.bh_total);  // heaviest causal tiles first
  const int q0 = qt * kBwdRows;
  const int i_row = q0 + 32 * wid + ql;
  const bool qvalid = i_row < n;
  const int lim = !qvalid ? 0 : (a.causal ? i_row + 1 : n);
  const int kend = a.causal ? min(n, q0 + kBwdRows) : n;
  const int ntiles = (kend + 31) / 32;
  const int wq0 = q0 + 32 * wid;
  const int wlim = wq0 >= n ? 0 : (a.causal ? min(n, wq0 + 32) : n);
  const int wtiles = (wlim + 31) / 32;

  for (int t = tid; t <= d; t += kBwdThreads) wtab[t] = expf(-2.0f * a.scale * static_cast<float>(t));

  const int64_t row = bh * n + (qvalid ? i_row : 0);
  int T = 0, cut = -1, hmin = 0;
  float invZ = 0.0f;
  uint32_t qw[W];
  v8bf db[NC][3];  // dout[i_row][16c + 8 half + s] as hi, mid, lo (the B operand of dP)
  float D = 0.0f;
  {
    const int4 st = *reinterpret_cast<const int4*>(a.stats + row * 4);
    T = st.x;
    cut = st.y;
    hmin = st.z;
    const float Z = __builtin_bit_cast(float, st.w);
    invZ = (qvalid && Z > 0.0f) ? 1.0f / Z : 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) qw[w] = a.qbits[row * W + w];
    const float* drow = a.dout + row * d;
    const float* orow = a.out + row * d;
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float x[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int f = 16 * c + 8 * half + s;
        const bool in = qvalid && f < d;
        x[s] = in ? drow[in ? f : 0] : 0.0f;
        part = fmaf(x[s], in ? orow[in ? f : 0] : 0.0f, part);
      }
      split8(x, db[c]);
    }
    D = part + __shfl_xor(part, 32, 64);  // both halves of the row
  }
  if (qvalid && half == 0) a.dsum[row] = D;
  const int tcut = cut >= 0 ? ((T << 16) | cut) : ((T << 16) - 1);
  const float pscale = a.scale * invZ;

  v16f acc[W];
#pragma unroll
  for (int t = 0; t < W; ++t) acc[t] = v16f{};

  const uint32_t* kbase = a.kbits + bh * static_cast<int64_t>(n) * W;
  const uint16_t* vsrc = static_cast<const uint16_t*>(a.v) + bh * static_cast<int64_t>(n) * d;
  uint32_t pk = 0;
  uint16_t pv[kVPT];
  int staged_k0 = 0;
  auto prefetch = [&](int tile) {
    const int k0 = 32 * tile;
    staged_k0 = k0;
    pk = kbase[static_cast<int64_t>(min(k0 + min(tid, 32 * W - 1) / W, n - 1)) * W + tid % W];
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      const int e = tid + j * kBwdThreads;
      const int r = e / DP, f = e - r * DP;
      pv[j] = vsrc[static_cast<int64_t>(min(k0 + r, n - 1)) * d + min(f, d - 1)];
    }
  };
  auto commit = [&](int buf) {
    if (tid < 32 * W) kw[buf][tid] = pk;
#pragma unroll
    for (int j = 0; j < kVPT; ++j) {
      const int e = tid + j * kBwdThreads;
      const int r = e / DP, f = e - r * DP;
      vt[buf][r * VSB + f] = (staged_k0 + r < n && f < d) ? pv[j] : static_cast<uint16_t>(0);
    }
  };
  prefetch(0);
  commit(0);
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    const int k0 = 32 * tile;
    if (tile + 1 < ntiles) prefetch(tile + 1);
    if (tile < wtiles) {
      const uint32_t* kwb = kw[buf];
      uint32_t kwv[16][W];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int w = 0; w < W; ++w) kwv[i][w] = kwb[tile_row(i, half) * W + w];
      }
      // dP tile (rows = keys, columns = query rows): A = the V tile row of
      // key ql, features 16c + 8 half .. + 7
      v8bf va[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        va[c] = __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(&vt[buf][ql * VSB + 16 * c + 8 * half]));
      // scale * p: kept iff visible and (h, key) <= (T, cut) in the order of
      // h << 16 | key (keys < 2^16); the table index h - h_min is clamped as
      // unsigned (a hidden key may lie below h_min)
      float sp[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + tile_row(i, half);
        int h = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) h += __builtin_popcount(qw[w] ^ kwv[i][w]);
        const bool keep = (((h << 16) | key) <= tcut) & (key < lim);
        const float wt = wtab[min(static_cast<uint32_t>(h - hmin), static_cast<uint32_t>(d))];
        sp[i] = keep ? wt * pscale : 0.0f;
      }
      v16f dp = v16f{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        dp = MFMA_BF16(va[c], db[c][0], dp);
        dp = MFMA_BF16(va[c], db[c][1], dp);
        dp = MFMA_BF16(va[c], db[c][2], dp);
      }
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = sp[i] * (dp[i] - D);
      // dQ^T += Bk^T dS: slot (half, s) of step cc is the key tile_row(8cc + s, half)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        v8bf b[3];
        split8(ds + 8 * cc, b);
#pragma unroll
        for (int t = 0; t < W; ++t) {
          uint32_t wsel[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) wsel[s] = kwv[8 * cc + s][t];
          const v8bf sa = sign_operand(wsel, ql);
          acc[t] = MFMA_BF16(sa, b[0], acc[t]);
          acc[t] = MFMA_BF16(sa, b[1], acc[t]);
          acc[t] = MFMA_BF16(sa, b[2], acc[t]);
        }
      }
    }
    if (tile + 1 < ntiles) commit(buf ^ 1);
    __syncthreads();
  }
  if (!qvalid) return;
  const float g = a.sigma_q != nullptr ? 1.0f / *a.sigma_q : 1.0f;
  float* drow = a.dq + row * d;
#pragma unroll
  for (int t = 0; t < W; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int f = 32 * t + tile_row(i, half);
      if (f < d) drow[f] = acc[t][i] * g;
    }
  }
}

// ---- 3. dK and dV (key-major) ----------------------------------------------
// Tiles of 32 query rows (sign words, dout rows, row statistics, D) staged
// double-buffered as in the dQ launch.  The key's V row, the B operand of
// dP, is held as float32 (fp32 V) or as packed bf16 pairs (bf16 V).
template <int W, bool VF32>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkv_kernel(BwdArgs a) {
  constexpr int DP = 32 * W;
  constexpr int OS = DP + 1;  // LDS row stride of the dout tile
  constexpr int kOPT = DP / 8;  // dout values per thread per tile
  constexpr int kVR = VF32 ? 16 * W : 8 * W;  // registers of the key's V row
  __shared__ float ot[2][32 * OS];
  __shared__ uint32_t qwt[2][32 * W];
  __shared__ int4 qst[2][32];    // T, last kept tie, h_min, 1/Z bits
  __shared__ float qd[2][32];    // D
  __shared__ float wtab[DP + 1];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, kl = lane & 31;
  const int n = a.n, d = a.d;
  const int64_t bh = blockIdx.x % a.bh_total;
  // causal: the first key tiles see the most query rows; dispatch them first
  const int kt = static_cast<int>(blockIdx.x / a.bh_total);
  const int k0 = kt * kBwdRows;
  const int j = k0 + 32 * wid + kl;
  const bool kvalid = j < n;
  const int qstart = a.causal ? (k0 / 32) : 0;  // first query tile any key of the block sees
  const int ntiles = (n + 31) / 32;
  const int wk0 = k0 + 32 * wid;
  const int wfirst = a.causal ? (wk0 / 32) : 0;  // first query tile this wave sees
  const bool wactive = wk0 < n;

  for (int t = tid; t <= d; t += kBwdThreads) wtab[t] = expf(-2.0f * a.scale * static_cast<float>(t));

  const int64_t krow = bh * n + (kvalid ? j : 0);
  uint32_t kw[W];
  uint32_t vr[kVR];  // V[j][2s + half] for s < 16W: fp32 bits, or bf16 pairs (s even | s odd << 16)
#pragma unroll
  for (int w = 0; w < W; ++w) kw[w] = a.kbits[krow * W + w];
#pragma unroll
  for (int s = 0; s < 16 * W; ++s) {
    const int f = 2 * s + half;
    const float x = (kvalid && f < d) ? load_v(a.v, krow * d + f, VF32) : 0.0f;
    if constexpr (VF32) {
      vr[s] = __builtin_bit_cast(uint32_t, x);
    } else {
      const uint32_t b = __builtin_bit_cast(uint32_t, x) >> 16;  // exact: x is a bf16 value
      vr[s >> 1] = (s & 1) ? (vr[s >> 1] | (b << 16)) : b;
    }
  }
  auto vval = [&](int s) {
    if constexpr (VF32) return __builtin_bit_cast(float, vr[s]);
    else return __builtin_bit_cast(float, (s & 1) ? (vr[s >> 1] & 0xFFFF0000u) : (vr[s >> 1] << 16));
  };
  v16f accv[W], acck[W];
#pragma unroll
  for (int t = 0; t < W; ++t) {
    accv[t] = v16f{};
    acck[t] = v16f{};
  }

  const int64_t rbase = bh * static_cast<int64_t>(n);
  // unconditional loads from clamped addresses, out-of-range values zeroed
  // when written (all of a thread's loads in flight together)
  uint32_t pq = 0;
  float po[kOPT];
  int4 pst = make_int4(0, 0, 0, 0);
  float pd = 0.0f;
  int staged_r0 = 0;
  auto prefetch = [&](int tile) {
    const int r0 = 32 * tile;
    staged_r0 = r0;
    pq = a.qbits[(rbase + min(r0 + min(tid, 32 * W - 1) / W, n - 1)) * W + tid % W];
#pragma unroll
    for (int jj = 0; jj < kOPT; ++jj) {
      const int e = tid + jj * kBwdThreads;
      const int r = e / DP, f = e - r * DP;
      po[jj] = a.dout[(rbase + min(r0 + r, n - 1)) * d + min(f, d - 1)];
    }
    const int q = min(r0 + (tid & 31), n - 1);
    pst = *reinterpret_cast<const int4*>(a.stats + (rbase + q) * 4);
    pd = a.dsum[rbase + q];
  };
  auto commit = [&](int buf) {
    if (tid < 32 * W) qwt[buf][tid] = pq;
#pragma unroll
    for (int jj = 0; jj < kOPT; ++jj) {
      const int e = tid + jj * kBwdThreads;
      const int r = e / DP, f = e - r * DP;
      ot[buf][r * OS + f] = (staged_r0 + r < n && f < d) ? po[jj] : 0.0f;
    }
    if (tid < 32) {
      const float Z = __builtin_bit_cast(float, pst.w);
      qst[buf][tid] = make_int4(pst.x, pst.y, pst.z, __builtin_bit_cast(int32_t, Z > 0.0f ? 1.0f / Z : 0.0f));
      qd[buf][tid] = pd;
    }
  };
  if (qstart < ntiles) {
    prefetch(qstart);
    commit(0);
  }
  __syncthreads();
  for (int tile = qstart; tile < ntiles; ++tile) {
    const int buf = (tile - qstart) & 1;
    const int r0 = 32 * tile;
    if (tile + 1 < ntiles) prefetch(tile + 1);
    if (wactive && tile >= wfirst) {
      const float* otb = ot[buf];
      const uint32_t* qwb = qwt[buf];
      // the 16 query rows' words (also the +-1 operand of dS^T Bq below),
      // distances and weights, branch-free so that the LDS reads issue together
      uint32_t qwv[16][W];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int w = 0; w < W; ++w) qwv[i][w] = qwb[tile_row(i, half) * W + w];
      }
      float p[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rl = tile_row(i, half);
        const int q = r0 + rl;
        int h = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) h += __builtin_popcount(qwv[i][w] ^ kw[w]);
        const int4 st = qst[buf][rl];
        const bool vis = kvalid & (q < n) & (!a.causal | (j <= q));
        const bool keep = vis & ((h < st.x) | ((h == st.x) & (j <= st.y)));
        const float wt = wtab[min(max(h - st.z, 0), d)];
        p[i] = keep ? wt * __builtin_bit_cast(float, st.w) : 0.0f;
      }
      // dP tile: rows = query rows, columns = keys; A operands read 8 ahead
      v16f dp = v16f{};
      constexpr int kS = 16 * W;
      float va[2][8];
#pragma unroll
      for (int k = 0; k < 8; ++k) va[0][k] = otb[kl * OS + 2 * k + half];
#pragma unroll
      for (int c = 0; c < kS / 8; ++c) {
        if (c + 1 < kS / 8) {
#pragma unroll
          for (int k = 0; k < 8; ++k) va[(c + 1) & 1][k] = otb[kl * OS + 2 * (8 * (c + 1) + k) + half];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
          dp = __builtin_amdgcn_mfma_f32_32x32x2f32(va[c & 1][k], vval(8 * c + k), dp, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) dsv[i] = a.scale * p[i] * (dp[i] - qd[buf][tile_row(i, half)]);
      // dV^T += dout^T P and dK^T += Bq^T dS: A = feature 32t + kl of query
      // row tile_row(i, half); 2W independent chains, the dout operands of
      // the next row read while the current row's products run
      float ov[2][W];
#pragma unroll
      for (int t = 0; t < W; ++t) ov[0][t] = otb[tile_row(0, half) * OS + 32 * t + kl];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + 1 < 16) {
#pragma unroll
          for (int t = 0; t < W; ++t) ov[(i + 1) & 1][t] = otb[tile_row(i + 1, half) * OS + 32 * t + kl];
        }
#pragma unroll
        for (int t = 0; t < W; ++t) {
          accv[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(ov[i & 1][t], p[i], accv[t], 0, 0, 0);
          const float b = ((qwv[i][t] >> kl) & 1u) ? -1.0f : 1.0f;
          acck[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(b, dsv[i], acck[t], 0, 0, 0);
        }
      }
    }
    if (tile + 1 < ntiles) commit(buf ^ 1);
    __syncthreads();
  }
  if (!kvalid) return;
  const float g = a.sigma_k != nullptr ? 1.0f / *a.sigma_k : 1.0f;
  float* vrow = a.dv + krow * d;
  float* krow_out = a.dk + krow * d;
#pragma unroll
  for (int t = 0; t < W; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int f = 32 * t + tile_row(i, half);
      if (f < d) {
        vrow[f] = accv[t][i];
        krow_out[f] = acck[t][i] * g;
      }
    }
  }
}

// dK and dV, key-major, bf16 V.  As bwd_dkv_kernel; each dout tile
// is staged split (hi, mid, lo) twice: row-major for the A operand of dP
// (16 features of one query row per lane) and feature-major for the A
// operand of dV^T += dout^T P (for one feature, the 8 query rows whose
// weights the lane holds).  The key's V row stays in registers as bf16
// operands.  Products per tile: dP 3 per 16 features, dV 6 and dK 3 per 16
// query rows and 32 features.
template <int W>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(W == 2 ? 2 : 1))) void bwd_dkv_bf_kernel(BwdArgs a) {
  static_assert(W <= 4, "d <= 128");
  constexpr int DP = 32 * W;
  constexpr int NC = DP / 16;
  constexpr int OSB = DP + 8;       // row-major tile stride (bf16): 16-byte rows, odd multiple
  constexpr int TSB = 32 + 4;       // feature-major tile stride (bf16): 72-byte rows, so the 32
                                    // lanes' 8-byte reads of a column spread over the banks
  __shared__ __attribute__((aligned(16))) uint16_t ob[2][3][32 * OSB];
  __shared__ __attribute__((aligned(16))) uint16_t obt[2][3][DP * TSB];
  __shared__ __attribute__((aligned(8))) uint32_t qwt[2][32 * W];
  __shared__ int4 qst[2][32];    // (h << 16 | key) bound, h_min, 1/Z bits, D bits
  __shared__ float wtab[DP + 1];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, kl = lane & 31;
  const int n = a.n, d = a.d;
  const int64_t bh = blockIdx.x % a.bh_total;
  const int kt = static_cast<int>(blockIdx.x / a.bh_total);
  const int k0 = kt * kBwdRows;
  const int j = k0 + 32 * wid + kl;
  const bool kvalid = j < n;
  const int qstart = a.causal ? (k0 / 32) : 0;
  const int ntiles = (n + 31) / 32;
  const int wk0 = k0 + 32 * wid;
  const int wfirst = a.causal ? (wk0 / 32) : 0;
  const bool wactive = wk0 < n;

  for (int t = tid; t <= d; t += kBwdThreads) wtab[t] = expf(-2.0f * a.scale * static_cast<float>(t));

  const int64_t krow = bh * n + (kvalid ? j : 0);
  uint32_t kw[W];
#pragma unroll
  for (int w = 0; w < W; ++w) kw[w] = a.kbits[krow * W + w];
  // the key's V row, features 16c + 8 half + s (the B operand of dP; exact in bf16)
  v8bf vb[NC];
  {
    const uint16_t* vr = static_cast<const uint16_t*>(a.v) + krow * d;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int f = 16 * c + 8 * half + 2 * k;
        const uint32_t lo = (kvalid && f < d) ? vr[f] : 0u;
        const uint32_t hi = (kvalid && f + 1 < d) ? vr[f + 1] : 0u;
        u[k] = lo | (hi << 16);
      }
      vb[c] = __builtin_bit_cast(v8bf, u);
    }
  }
  v16f accv[W], acck[W];
#pragma unroll
  for (int t = 0; t < W; ++t) {
    accv[t] = v16f{};
    acck[t] = v16f{};
  }

  const int64_t rbase = bh * static_cast<int64_t>(n);
  // staging share: item e (4 DP of them) is features 2 (e % (DP/2)) and
  // + 1 of query rows 4 (e / (DP/2)) .. + 3; thread t takes items t, t + 256,
  // ...  The split terms of two features of a row (row-major planes) or of
  // two rows of a feature (feature-major planes) go into one dword.
  constexpr int kItems = (4 * DP + kBwdThreads - 1) / kBwdThreads;
  uint32_t pq = 0;
  float po[kItems][4][2];
  int4 pst = make_int4(0, 0, 0, 0);
  float pd = 0.0f;
  int staged_r0 = 0;
  auto prefetch = [&](int tile) {
    const int r0 = 32 * tile;
    staged_r0 = r0;
    pq = a.qbits[(rbase + min(r0 + min(tid, 32 * W - 1) / W, n - 1)) * W + tid % W];
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int e = min(tid + it * kBwdThreads, 4 * DP - 1);
      const int f0 = 2 * (e % (DP / 2)), sr0 = 4 * (e / (DP / 2));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t ro = (rbase + min(r0 + sr0 + u, n - 1)) * d;
        po[it][u][0] = a.dout[ro + min(f0, d - 1)];
        po[it][u][1] = a.dout[ro + min(f0 + 1, d - 1)];
      }
    }
    const int q = min(r0 + (tid & 31), n - 1);
    pst = *reinterpret_cast<const int4*>(a.stats + (rbase + q) * 4);
    pd = a.dsum[rbase + q];
  };
  auto commit = [&](int buf) {
    if (tid < 32 * W) qwt[buf][tid] = pq;
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int e = tid + it * kBwdThreads;
      if (e >= 4 * DP) break;
      const int f0 = 2 * (e % (DP / 2)), sr0 = 4 * (e / (DP / 2));
      // the three split terms of each value, as float32 words whose top
      // halves are the bf16 terms
      uint32_t t3[3][4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bool in = staged_r0 + sr0 + u < n && f0 + c < d;
          const float x = in ? po[it][u][c] : 0.0f;
          const uint32_t ux = __builtin_bit_cast(uint32_t, x);
          const float r = x - __builtin_bit_cast(float, ux & 0xFFFF0000u);
          const uint32_t ur = __builtin_bit_cast(uint32_t, r);
          const float l = r - __builtin_bit_cast(float, ur & 0xFFFF0000u);
          t3[0][u][c] = ux;
          t3[1][u][c] = ur;
          t3[2][u][c] = __builtin_bit_cast(uint32_t, l);
        }
      }
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          *reinterpret_cast<uint32_t*>(&ob[buf][pp][(sr0 + u) * OSB + f0]) =
              __builtin_amdgcn_perm(t3[pp][u][1], t3[pp][u][0], 0x07060302u);
#pragma unroll
        for (int c = 0; c < 2; ++c)
          *reinterpret_cast<uint2*>(&obt[buf][pp][(f0 + c) * TSB + sr0]) =
              make_uint2(__builtin_amdgcn_perm(t3[pp][1][c], t3[pp][0][c], 0x07060302u),
                         __builtin_amdgcn_perm(t3[pp][3][c], t3[pp][2][c], 0x07060302u));
      }
    }
    if (tid < 32) {
      // (h << 16 | key) bound of the row's kept keys (none for rows past the
      // end), h_min, 1/Z, D
      const float Z = __builtin_bit_cast(float, pst.w);
      const int tc = staged_r0 + tid >= n ? -1 : (pst.y >= 0 ? ((pst.x << 16) | pst.y) : ((pst.x << 16) - 1));
      qst[buf][tid] = make_int4(tc, pst.z, __builtin_bit_cast(int32_t, Z > 0.0f ? 1.0f / Z : 0.0f),
                                __builtin_bit_cast(int32_t, pd));
    }
  };
  if (qstart < ntiles) {
    prefetch(qstart);
    commit(0);
  }
  __syncthreads();
  for (int tile = qstart; tile < ntiles; ++tile) {
    const int buf = (tile - qstart) & 1;
    const int r0 = 32 * tile;
    if (tile + 1 < ntiles) prefetch(tile + 1);
    if (wactive && tile >= wfirst) {
      const uint32_t* qwb = qwt[buf];
      uint32_t qwv[16][W];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (W % 2 == 0) {
#pragma unroll
          for (int w = 0; w < W; w += 2) {
            const uint2 x = *reinterpret_cast<const uint2*>(&qwb[tile_row(i, half) * W + w]);
            qwv[i][w] = x.x;
            qwv[i][w + 1] = x.y;
          }
        } else {
#pragma unroll
          for (int w = 0; w < W; ++w) qwv[i][w] = qwb[tile_row(i, half) * W + w];
        }
      }
      // kept iff visible and (h, j) <= (T, cut) in the order of h << 16 | j;
      // a lane past the end writes nothing, so its weights need no mask
      float p[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rl = tile_row(i, half);
        const int q = r0 + rl;
        int h = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) h += __builtin_popcount(qwv[i][w] ^ kw[w]);
        const int4 st = qst[buf][rl];
        const bool keep = (((h << 16) | j) <= st.x) & (!a.causal | (j <= q));
        const float wt = wtab[min(static_cast<uint32_t>(h - st.y), static_cast<uint32_t>(d))];
        p[i] = keep ? wt * __builtin_bit_cast(float, st.z) : 0.0f;
      }
      // dP tile (rows = query rows, columns = keys): A = row kl of the split
      // dout tile, features 16c + 8 half .. + 7, read step by step
      v16f dp = v16f{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
          const v8bf oa = __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(&ob[buf][pp][kl * OSB + 16 * c + 8 * half]));
          dp = MFMA_BF16(oa, vb[c], dp);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        dsv[i] = a.scale * p[i] * (dp[i] - __builtin_bit_cast(float, qst[buf][tile_row(i, half)].w));
      // slot (half, s) of step cc is the query row tile_row(8cc + s, half):
      // rows 16cc + 4 half + s (s < 4) and 16cc + 8 + 4 half + s - 4
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        v8bf pb[3], sb[3];
        split8(p + 8 * cc, pb);
        split8(dsv + 8 * cc, sb);
#pragma unroll
        for (int t = 0; t < W; ++t) {
          v8bf da[3];
#pragma unroll
          for (int pp = 0; pp < 3; ++pp) {
            const uint16_t* col = &obt[buf][pp][(32 * t + kl) * TSB + 16 * cc + 4 * half];
            const uint2 lo = *reinterpret_cast<const uint2*>(col);
            const uint2 hi = *reinterpret_cast<const uint2*>(col + 8);
            da[pp] = __builtin_bit_cast(v8bf, u32x4{lo.x, lo.y, hi.x, hi.y});
          }
          // dV^T += dout^T P: the six partial products above 2^-24
          accv[t] = MFMA_BF16(da[0], pb[0], accv[t]);
          accv[t] = MFMA_BF16(da[0], pb[1], accv[t]);
          accv[t] = MFMA_BF16(da[1], pb[0], accv[t]);
          accv[t] = MFMA_BF16(da[0], pb[2], accv[t]);
          accv[t] = MFMA_BF16(da[1], pb[1], accv[t]);
          accv[t] = MFMA_BF16(da[2], pb[0], accv[t]);
          // dK^T += Bq^T dS
          uint32_t wsel[8];
#pragma unroll
          for (int s2 = 0; s2 < 8; ++s2) wsel[s2] = qwv[8 * cc + s2][t];
          const v8bf sa = sign_operand(wsel, kl);
          acck[t] = MFMA_BF16(sa, sb[0], acck[t]);
          acck[t] = MFMA_BF16(sa, sb[1], acck[t]);
          acck[t] = MFMA_BF16(sa, sb[2], acck[t]);
        }
      }
    }
    if (tile + 1 < ntiles) commit(buf ^ 1);
    __syncthreads();
  }
  if (!kvalid) return;
  const float g = a.sigma_k != nullptr ? 1.0f / *a.sigma_k : 1.0f;
  float* vrow = a.dv + krow * d;
  float* krow_out = a.dk + krow * d;
#pragma unroll
  for (int t = 0; t < W; ++t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int f = 32 * t + tile_row(i, half);
      if (f < d) {
        vrow[f] = accv[t][i];
        krow_out[f] = acck[t][i] * g;
      }
    }
  }
}

// Launches 2 and 3 for W words per row.
template <int W>
had_status launch_bwd(const BwdArgs& a, bool vf32, unsigned blocks, hipStream_t hs) {
  if (!vf32) {
    bwd_dq_bf_kernel<W><<<blocks, kBwdThreads, 0, hs>>>(a);
    had_status st = check_launch("had_backward");
    if (st != HAD_OK) return st;
    bwd_dkv_bf_kernel<W><<<blocks, kBwdThreads, 0, hs>>>(a);
    return check_launch("had_backward");
  }
  bwd_dq_kernel<W, true><<<blocks, kBwdThreads, 0, hs>>>(a);
  had_status st = check_launch("had_backward");
  if (st != HAD_OK) return st;
  bwd_dkv_kernel<W, true><<<blocks, kBwdThreads, 0, hs>>>(a);
  return check_launch("had_backward");
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace
}  // namespace had

using namespace had;

extern "C" size_t had_backward_workspace_bytes(had_shape s) {
  if (check_shape(s) != HAD_OK || s.dim > 128) return 0;
  const size_t rows = static_cast<size_t>(s.batch * s.heads * s.seq);
  return align256(rows * 4 * sizeof(int32_t)) + align256(rows * sizeof(float));
}

extern "C" had_status had_backward(const uint32_t* qbits, const uint32_t* kbits, const void* v,
                                   had_dtype v_dtype, had_shape s, int64_t topn, float scale,
                                   int causal, const float* out, const float* dout,
                                   const float* sigma_q, const float* sigma_k, float* dq, float* dk,
                                   float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  had_status st = check_shape(s);
  if (st != HAD_OK) return st;
  if (s.dim > 128) return fail(HAD_ERR_UNSUPPORTED, "had_backward: dim above 128");
  if (qbits == nullptr || kbits == nullptr || v == nullptr || out == nullptr || dout == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return fail(HAD_ERR_INVALID_ARG, "had_backward: null pointer argument");
  if (!aligned(qbits, 4) || !aligned(kbits, 4) || !aligned(v, 4) || !aligned(out, 4) ||
      !aligned(dout, 4) || !aligned(dq, 4) || !aligned(dk, 4) || !aligned(dv, 4))
    return fail(HAD_ERR_INVALID_ARG, "had_backward: pointers must be 4-byte aligned");
  if ((sigma_q != nullptr && !aligned(sigma_q, 4)) || (sigma_k != nullptr && !aligned(sigma_k, 4)))
    return fail(HAD_ERR_INVALID_ARG, "had_backward: sigma pointers must be 4-byte aligned");
  const int vdt = enum_bits(v_dtype);
  if (!valid_dtype(vdt)) return fail(HAD_ERR_INVALID_ARG, "had_backward: unknown v_dtype");
  if (topn < 1) return fail(HAD_ERR_INVALID_ARG, "had_backward: topn must be >= 1");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(HAD_ERR_INVALID_ARG, "had_backward: scale must be finite and > 0");
  if (causal != 0 && causal != 1) return fail(HAD_ERR_INVALID_ARG, "had_backward: causal must be 0 or 1");
  if (workspace == nullptr || !aligned(workspace, 256))
    return fail(HAD_ERR_INVALID_ARG, "had_backward: workspace must be non-null and 256-byte aligned");
  if (workspace_bytes < had_backward_workspace_bytes(s))
    return fail(HAD_ERR_INVALID_ARG, "had_backward: workspace smaller than had_backward_workspace_bytes()");
  const int64_t bh = s.batch * s.heads;
  const size_t rows = static_cast<size_t>(bh * s.seq);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  int32_t* stats = reinterpret_cast<int32_t*>(ws);
  float* dsum = reinterpret_cast<float*>(ws + align256(rows * 4 * sizeof(int32_t)));
  hipStream_t hs = static_cast<hipStream_t>(stream);

  // 1. row statistics (the attention kernel's histogram pass)
  AttnArgs sa{};
  sa.qbits = qbits;
  sa.kbits = kbits;
  sa.v_dtype = HAD_BF16;
  sa.bh_total = bh;
  sa.bh_begin = 0;
  sa.bh_count = bh;
  sa.n = static_cast<int>(s.seq);
  sa.d = static_cast<int>(s.dim);
  sa.topn = static_cast<int>(topn > s.seq ? s.seq : topn);
  sa.scale = scale;
  sa.causal = causal;
  sa.rowstats = stats;
  if ((st = launch_attention_family(AttnMode::Stats, sa, hs)) != HAD_OK) return st;

  BwdArgs a{};
  a.qbits = qbits;
  a.kbits = kbits;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.sigma_q = sigma_q;
  a.sigma_k = sigma_k;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.stats = stats;
  a.dsum = dsum;
  a.bh_total = bh;
  a.n = static_cast<int>(s.seq);
  a.d = static_cast<int>(s.dim);
  a.scale = scale;
  a.causal = causal;
  const int64_t blocks = ((s.seq + kBwdRows - 1) / kBwdRows) * bh;
  if (blocks > 0x7FFFFFFF) return fail(HAD_ERR_UNSUPPORTED, "had_backward: grid too large");
  const unsigned nb = static_cast<unsigned>(blocks);
  const bool vf32 = vdt == HAD_F32;
  switch (words_per_row(s.dim)) {
    case 1: return launch_bwd<1>(a, vf32, nb, hs);
    case 2: return launch_bwd<2>(a, vf32, nb, hs);
    case 3: return launch_bwd<3>(a, vf32, nb, hs);
    case 4: return launch_bwd<4>(a, vf32, nb, hs);
  }
  return fail(HAD_ERR_UNSUPPORTED, "had_backward: dim above 128");
}
