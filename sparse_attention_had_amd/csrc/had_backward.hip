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
// Everything is float32 on the matrix cores (their fp32 products round like
// the vector ALU's); no floating-point atomics, so results are identical run
// to run.  Masked elements take weight 0.
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
template <int W, bool VF32>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(BwdArgs a) {
  constexpr int DP = 32 * W;   // padded features
  constexpr int VS = DP + 1;   // LDS row stride of the V tile (no bank conflicts)
  __shared__ float vt[32 * VS];
  __shared__ uint32_t kw[32 * W];
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
  for (int tile = 0; tile < ntiles; ++tile) {
    const int k0 = 32 * tile;
    __syncthreads();  // the previous tile is consumed
    for (int e = tid; e < 32 * W; e += kBwdThreads) {
      const int key = min(k0 + e / W, n - 1);
      kw[e] = kbase[static_cast<int64_t>(key) * W + e % W];
    }
    for (int e = tid; e < 32 * DP; e += kBwdThreads) {
      const int r = e / DP, f = e - r * DP;
      const int key = k0 + r;
      vt[r * VS + f] = (key < n && f < d) ? load_v(a.v, vbase + static_cast<int64_t>(key) * d + f, VF32) : 0.0f;
    }
    __syncthreads();
    if (tile >= wtiles) continue;
    // weights of this lane's 16 keys (zero where not kept)
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kl = tile_row(i, half);
      const int key = k0 + kl;
      int h = 0;
#pragma unroll
      for (int w = 0; w < W; ++w) h += __builtin_popcount(qw[w] ^ kw[kl * W + w]);
      const bool keep = key < lim && (h < T || (h == T && key <= cut));
      p[i] = keep ? wtab[min(max(h - hmin, 0), d)] * invZ : 0.0f;
    }
    // dP tile: rows = keys, columns = query rows
    v16f dp = v16f{};
#pragma unroll
    for (int s = 0; s < 16 * W; ++s)
      dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vt[ql * VS + 2 * s + half], dr[s], dp, 0, 0, 0);
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ds[i] = a.scale * p[i] * (dp[i] - D);
    // dQ^T += Bk^T dS: A = +-1 of feature 32t + ql of key tile_row(i, half)
#pragma unroll
    for (int t = 0; t < W; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t word = kw[tile_row(i, half) * W + t];
        const float b = ((word >> ql) & 1u) ? -1.0f : 1.0f;
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(b, ds[i], acc[t], 0, 0, 0);
      }
    }
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
template <int W, bool VF32>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkv_kernel(BwdArgs a) {
  constexpr int DP = 32 * W;
  constexpr int OS = DP + 1;  // LDS row stride of the dout tile
  __shared__ float ot[32 * OS];
  __shared__ uint32_t qwt[32 * W];
  __shared__ int4 qst[32];    // T, last kept tie, h_min, 1/Z bits
  __shared__ float qd[32];    // D
  __shared__ float wtab[DP + 1];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5, kl = lane & 31;
  const int n = a.n, d = a.d;
  const int ntk = (n + kBwdRows - 1) / kBwdRows;
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
  float vr[16 * W];  // V[j][2s + half] (the B operand of dP)
#pragma unroll
  for (int w = 0; w < W; ++w) kw[w] = a.kbits[krow * W + w];
#pragma unroll
  for (int s = 0; s < 16 * W; ++s) {
    const int f = 2 * s + half;
    vr[s] = (kvalid && f < d) ? load_v(a.v, krow * d + f, VF32) : 0.0f;
  }
  v16f accv[W], acck[W];
#pragma unroll
  for (int t = 0; t < W; ++t) {
    accv[t] = v16f{};
    acck[t] = v16f{};
  }

  const int64_t rbase = bh * static_cast<int64_t>(n);
  for (int tile = qstart; tile < ntiles; ++tile) {
    const int r0 = 32 * tile;
    __syncthreads();
    for (int e = tid; e < 32 * W; e += kBwdThreads) {
      const int q = min(r0 + e / W, n - 1);
      qwt[e] = a.qbits[(rbase + q) * W + e % W];
    }
    for (int e = tid; e < 32 * DP; e += kBwdThreads) {
      const int r = e / DP, f = e - r * DP;
      const int q = r0 + r;
      ot[r * OS + f] = (q < n && f < d) ? a.dout[(rbase + q) * d + f] : 0.0f;
    }
    if (tid < 32) {
      const int q = min(r0 + tid, n - 1);
      const int4 st = *reinterpret_cast<const int4*>(a.stats + (rbase + q) * 4);
      const float Z = __builtin_bit_cast(float, st.w);
      qst[tid] = make_int4(st.x, st.y, st.z, __builtin_bit_cast(int32_t, Z > 0.0f ? 1.0f / Z : 0.0f));
      qd[tid] = a.dsum[rbase + q];
    }
    __syncthreads();
    if (!wactive || tile < wfirst) continue;
    float p[16], dsv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rl = tile_row(i, half);
      const int q = r0 + rl;
      int h = 0;
#pragma unroll
      for (int w = 0; w < W; ++w) h += __builtin_popcount(qwt[rl * W + w] ^ kw[w]);
      const int4 st = qst[rl];
      const bool vis = kvalid && q < n && (!a.causal || j <= q);
      const bool keep = vis && (h < st.x || (h == st.x && j <= st.y));
      p[i] = keep ? wtab[min(max(h - st.z, 0), d)] * __builtin_bit_cast(float, st.w) : 0.0f;
    }
    // dP tile: rows = query rows, columns = keys
    v16f dp = v16f{};
#pragma unroll
    for (int s = 0; s < 16 * W; ++s)
      dp = __builtin_amdgcn_mfma_f32_32x32x2f32(ot[kl * OS + 2 * s + half], vr[s], dp, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) dsv[i] = a.scale * p[i] * (dp[i] - qd[tile_row(i, half)]);
    // dV^T += dout^T P and dK^T += Bq^T dS: A = feature 32t + kl of query row tile_row(i, half)
#pragma unroll
    for (int t = 0; t < W; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rl = tile_row(i, half);
        accv[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(ot[rl * OS + 32 * t + kl], p[i], accv[t], 0, 0, 0);
        const float b = ((qwt[rl * W + t] >> kl) & 1u) ? -1.0f : 1.0f;
        acck[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(b, dsv[i], acck[t], 0, 0, 0);
      }
    }
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
  if (vf32)
    bwd_dq_kernel<W, true><<<blocks, kBwdThreads, 0, hs>>>(a);
  else
    bwd_dq_kernel<W, false><<<blocks, kBwdThreads, 0, hs>>>(a);
  had_status st = check_launch("had_backward");
  if (st != HAD_OK) return st;
  if (vf32)
    bwd_dkv_kernel<W, true><<<blocks, kBwdThreads, 0, hs>>>(a);
  else
    bwd_dkv_kernel<W, false><<<blocks, kBwdThreads, 0, hs>>>(a);
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
