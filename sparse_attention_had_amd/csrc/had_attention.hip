// had_attention / had_select / had_logits: the fused HAD attention kernel.
//
// Method (Pith review of "Hamming Attention Distillation", section "What
// carries the argument"; verdict record "one_line_summary"): integer logits
// s = d - 2*popcount(q XOR k) of the sign-binarized rows, a top-N mask that
// keeps the largest logits of each query row, softmax over the kept logits,
// and the weighted sum of full-precision V rows.  Lower key index wins among
// equal logits; a causal mask (row i sees keys j <= i) is applied before the
// selection.
//
// GPU design (gfx950 / CDNA4), one work-group = WAVES waves x 32 query rows of
// one (batch, head) slice; the n x n matrix never leaves the registers.
//
//  * Logits on the int8 matrix cores.  Sign bits are expanded to +-1 bytes
//    (K: once per block per key chunk into LDS; Q: once per wave into
//    registers) and v_mfma_i32_32x32x32_i8 computes S^T = K Q^T, exactly,
//    32 keys x 32 queries per instruction and 32 features of d.
//  * Key order.  The block's visible key range [0, kend) is split at Hh into
//    two halves.  In the S^T tile the output registers i = 0..15 of lane L hold
//    query L%32 and keys half*Hh + 16*chunk + i with half = L/32, so every lane
//    walks its half of the keys in ascending order.  "Lower index wins" among
//    the tied keys then reduces to a per-lane running quota.
//  * Selection, pass 1.  Per-wave LDS histogram over the d+1 possible logits:
//    dword [bin][query] holds the half-0 count in its low and the half-1
//    count in its high 16 bits (ds_add_u32 of 1 or 1<<16; the two lane halves
//    run in separate LDS cycles, 32 distinct queries per cycle = 32 banks).
//    A scan per row gives the threshold bin T, the tie quota r split over the
//    halves, h_min and the softmax denominator Z (from counts, without V).
//  * Pass 2.  The logits are recomputed on the matrix cores (cheaper than
//    storing them), each element is kept or dropped, its weight
//    exp(-2*scale*(h - h_min)) is read from an LDS table as a pair of bf16
//    terms (hi + lo, relative error < 2^-15), and out^T = V^T P^T runs on
//    v_mfma_f32_32x32x16_bf16 (two products, hi and lo) with V staged
//    transposed in LDS.  fp32 V uses v_mfma_f32_32x32x2_f32 with fp32 weights.
//    Dense-masked products on the matrix cores beat a per-row gather of the
//    N kept V rows: a gather reads 2*d bytes of on-chip bandwidth per kept
//    pair, the tile product reuses every staged V row for 32 query rows.
#include "had_internal.h"

namespace had {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCH = 2;          // 16-key chunks per half staged per iteration
constexpr int kLutEntries = 264;  // weight table: d+1 weights + zero slot
constexpr int kZeroSlot = 263;

template <int W>
struct Cfg {
  static constexpr int kWaves = (W <= 2) ? 4 : (W <= 4 ? 2 : 1);
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kQB = 32 * kWaves;    // query rows per block
  static constexpr int kDP = 32 * W;         // padded feature count
  static constexpr int kKxStride = kDP + 16;  // bytes per expanded key row
};

__host__ __device__ constexpr int vt_stride_bytes(bool vf32) { return vf32 ? 144 : 80; }

template <int W, bool VF32>
__host__ __device__ constexpr size_t lds_layout_kx() {
  return 2048 + 4 * kLutEntries;  // after byte table and weight table
}

template <int W, bool VF32>
__host__ __device__ constexpr size_t lds_layout_region() {
  return lds_layout_kx<W, VF32>() + static_cast<size_t>(kCH) * 32 * Cfg<W>::kKxStride;
}

template <int W, bool VF32>
size_t lds_bytes(int d) {
  const size_t hist = static_cast<size_t>(Cfg<W>::kWaves) * (d + 1) * 32 * 4;
  const size_t vt = static_cast<size_t>(kCH) * Cfg<W>::kDP * vt_stride_bytes(VF32);
  return lds_layout_region<W, VF32>() + (hist > vt ? hist : vt);
}

__device__ inline uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ inline float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t u = f2u(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ inline float bf16_to_f(uint32_t b) { return u2f(b << 16); }

// 4 sign bits -> 4 int8 lanes of +1 (bit 0) / -1 (bit 1).
__device__ inline uint32_t expand_nibble(uint32_t nib) {
  const uint32_t y = (nib * 0x00204081u) & 0x01010101u;  // bit k -> byte k
  return (y * 0xFEu) | 0x01010101u;
}

// Byte mask keeping the d-elements [base, base+4) that are < d.
__device__ inline uint32_t pad_mask4(int base, int d) {
  const int valid = d - base;
  if (valid >= 4) return 0xFFFFFFFFu;
  if (valid <= 0) return 0u;
  return (1u << (8 * valid)) - 1u;
}

template <int W, bool VF32, int MODE>
__global__ __launch_bounds__(Cfg<W>::kThreads) void had_attn_kernel(AttnArgs a) {
  using C = Cfg<W>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  uint2* byte_lut = reinterpret_cast<uint2*>(lds);                 // 256 x 8 B
  uint32_t* wlut = reinterpret_cast<uint32_t*>(lds + 2048);         // kLutEntries
  unsigned char* kx = lds + lds_layout_kx<W, VF32>();               // kCH x 32 x stride
  unsigned char* region = lds + lds_layout_region<W, VF32>();      // hist | vt

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int half = lane >> 5;
  const int ql = lane & 31;
  const int n = a.n;
  const int d = a.d;

  // ---- block -> (slice, query tile); heaviest causal tiles dispatch first
  const int qrows = (MODE == 2) ? a.row_count : n;
  const int ntq = (qrows + C::kQB - 1) / C::kQB;
  const int64_t bid = blockIdx.x;
  const int64_t bh_local = bid % a.bh_count;
  const int qt = ntq - 1 - static_cast<int>(bid / a.bh_count);
  const int64_t bh = a.bh_begin + bh_local;
  const int qbase = (MODE == 2) ? a.row_begin : 0;
  const int q0 = qbase + qt * C::kQB;
  const int qend = qbase + qrows;
  const int i_row = q0 + wid * 32 + ql;
  const bool qvalid = i_row < qend;
  const bool causal = (MODE != 2) && a.causal;

  const int kend = causal ? min(n, q0 + C::kQB) : n;
  const int Hh = ((kend + 1) / 2 + 15) & ~15;  // half split, multiple of 16
  const int nchunk = Hh / 16;
  const int niter = (nchunk + kCH - 1) / kCH;
  // keys j < lim are visible to this lane's query row
  const int lim = !qvalid ? 0 : (causal ? min(i_row + 1, n) : n);
  const int wave_q0 = q0 + wid * 32;
  const int wlim = (wave_q0 >= qend) ? 0 : (causal ? min(n, wave_q0 + 32) : n);

  // ---- constant tables
  for (int t = tid; t < 256; t += C::kThreads)
    byte_lut[t] = make_uint2(expand_nibble(t & 15u), expand_nibble(t >> 4));
  if (MODE == 0) {
    for (int t = tid; t < kLutEntries; t += C::kThreads) {
      uint32_t e = 0;
      if (t <= d) {
        const float w = expf(-2.0f * a.scale * static_cast<float>(t));
        if (VF32) {
          e = f2u(w);
        } else {
          const uint32_t hi = bf16_rne(w);
          const uint32_t lo = bf16_rne(w - bf16_to_f(hi));
          e = hi | (lo << 16);
        }
      }
      wlut[t] = e;
    }
  }

  // ---- Q operand: +-1 bytes of this lane's query, features 32w + 16*half + [0,16)
  v4i qx[W];
  {
    const uint32_t* qrow = a.qbits + (bh * n + (qvalid ? i_row : 0)) * W;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const uint32_t word = qvalid ? qrow[w] : 0u;
      const uint32_t b16 = (word >> (16 * half)) & 0xFFFFu;
      const int fbase = 32 * w + 16 * half;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        qx[w][k] = static_cast<int>(expand_nibble((b16 >> (4 * k)) & 15u) & pad_mask4(fbase + 4 * k, d));
    }
  }

  const uint32_t* kb = a.kbits + bh * static_cast<int64_t>(n) * W;

  // Stage the expanded keys of chunks [it*kCH, it*kCH + kCH) into kx.
  auto stage_k = [&](int it) {
    for (int item = tid; item < kCH * 32 * W; item += C::kThreads) {
      const int w = item % W;
      const int m = (item / W) & 31;
      const int c = item / (W * 32);
      const int gc = it * kCH + c;
      const int hf = (m >> 2) & 1;
      const int r = 4 * (m >> 3) + (m & 3);
      const int key = hf * Hh + 16 * gc + r;
      const uint32_t word = (gc < nchunk && key < kend) ? kb[static_cast<int64_t>(key) * W + w] : 0u;
      uint32_t o[8];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint2 e = byte_lut[(word >> (8 * b)) & 0xFFu];
        o[2 * b] = e.x & pad_mask4(32 * w + 8 * b, d);
        o[2 * b + 1] = e.y & pad_mask4(32 * w + 8 * b + 4, d);
      }
      u32x4* dst = reinterpret_cast<u32x4*>(kx + (c * 32 + m) * C::kKxStride + 32 * w);
      dst[0] = u32x4{o[0], o[1], o[2], o[3]};
      dst[1] = u32x4{o[4], o[5], o[6], o[7]};
    }
  };

  // S^T tile of chunk c: acc[i] = logit(query ql, key half*Hh + 16*gc + i).
  auto logits_tile = [&](int c) {
    v16i acc = {};
    const unsigned char* krow = kx + (c * 32 + ql) * C::kKxStride + 16 * half;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const v4i kv = *reinterpret_cast<const v4i*>(krow + 32 * w);
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kv, qx[w], acc, 0, 0, 0);
    }
    return acc;
  };

  // =========================================================== logits export
  if (MODE == 2) {
    for (int it = 0; it < niter; ++it) {
      __syncthreads();
      stage_k(it);
      __syncthreads();
      for (int c = 0; c < kCH; ++c) {
        const int gc = it * kCH + c;
        if (gc >= nchunk) break;
        const v16i s = logits_tile(c);
        if (!qvalid) continue;
        const int kbase = half * Hh + 16 * gc;
        int16_t* dst = a.logits + (bh_local * a.row_count + (i_row - a.row_begin)) * static_cast<int64_t>(n);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kbase + i < lim) dst[kbase + i] = static_cast<int16_t>(s[i]);
      }
    }
    return;
  }

  // =========================================================== pass 1: histogram
  uint32_t* hist = reinterpret_cast<uint32_t*>(region) + wid * (d + 1) * 32;
  for (int t = lane; t < (d + 1) * 32; t += 64) hist[t] = 0u;
  const uint32_t addend = half ? 0x10000u : 1u;

  for (int it = 0; it < niter; ++it) {
    __syncthreads();
    stage_k(it);
    __syncthreads();
    for (int c = 0; c < kCH; ++c) {
      const int gc = it * kCH + c;
      if (gc >= nchunk) break;
      if (16 * gc >= wlim) break;  // nothing visible to this wave any more
      const v16i s = logits_tile(c);
      const int L = lim - (half * Hh + 16 * gc);  // element i visible iff i < L
      uint32_t* hq = hist + ql;
      if (__all(L >= 16)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) atomicAdd(hq + ((d - s[i]) >> 1) * 32, addend);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i < L) atomicAdd(hq + ((d - s[i]) >> 1) * 32, addend);
      }
    }
  }
  __syncthreads();

  // =========================================================== per-row statistics
  const int Ni = qvalid ? min(a.topn, lim) : 0;
  int T = 0, hmin = 0, below0 = 0, ties0 = 0, below = 0;
  {
    const uint32_t* hq = hist + ql;
    int cum = 0, cum0 = 0;
    bool have_min = false;
    for (int b = 0; b <= d; ++b) {
      const uint32_t x = hq[b * 32];
      const int c0 = static_cast<int>(x & 0xFFFFu);
      const int cnt = c0 + static_cast<int>(x >> 16);
      if (!have_min && cnt > 0) {
        hmin = b;
        have_min = true;
      }
      if (cum + cnt >= Ni) {
        T = b;
        below = cum;
        below0 = cum0;
        ties0 = c0;
        break;
      }
      cum += cnt;
      cum0 += c0;
    }
  }
  const int r_tie = Ni - below;
  const int quota0 = min(r_tie, ties0);
  int quota = half ? (r_tie - quota0) : quota0;
  const int sT = (Ni > 0) ? d - 2 * T : d + 2;  // rows with nothing to keep never match

  if (MODE == 1) {
    // ======================================================= selection export
    int pos = half ? (below0 + quota0) : 0;
    int32_t* dst = a.idx + (bh_local * n + (qvalid ? i_row : 0)) * static_cast<int64_t>(a.topn);
    for (int it = 0; it < niter; ++it) {
      __syncthreads();
      stage_k(it);
      __syncthreads();
      for (int c = 0; c < kCH; ++c) {
        const int gc = it * kCH + c;
        if (gc >= nchunk) break;
        if (16 * gc >= wlim) break;
        const v16i s = logits_tile(c);
        const int kbase = half * Hh + 16 * gc;
        const int L = lim - kbase;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool valid = i < L;
          const bool eq = valid && (s[i] == sT);
          const bool keep = (valid && s[i] > sT) || (eq && quota > 0);
          quota -= eq ? 1 : 0;
          if (keep && pos < a.topn) dst[pos++] = kbase + i;
        }
      }
    }
    if (qvalid && half == 0)
      for (int p = Ni; p < a.topn; ++p) dst[p] = -1;
    return;
  }

  // =========================================================== pass 2: attend
  float Z = 0.0f;
  if (Ni > 0) {
    const uint32_t* hq = hist + ql;
    for (int b = hmin; b < T; ++b) {
      const uint32_t x = hq[b * 32];
      const int cnt = static_cast<int>(x & 0xFFFFu) + static_cast<int>(x >> 16);
      const uint32_t e = wlut[b - hmin];
      const float w = VF32 ? u2f(e) : bf16_to_f(e & 0xFFFFu) + bf16_to_f(e >> 16);
      Z += static_cast<float>(cnt) * w;
    }
    const uint32_t e = wlut[T - hmin];
    const float w = VF32 ? u2f(e) : bf16_to_f(e & 0xFFFFu) + bf16_to_f(e >> 16);
    Z += static_cast<float>(r_tie) * w;
  }
  const float invZ = (Z > 0.0f) ? 1.0f / Z : 0.0f;
  // weight-table index of logit s: (d - s)/2 - hmin
  const int lut_off = d - 2 * hmin;

  v16f acc[W];
#pragma unroll
  for (int t = 0; t < W; ++t) acc[t] = v16f{};

  const unsigned char* vsrc = static_cast<const unsigned char*>(a.v) +
                              bh * static_cast<int64_t>(n) * d * (VF32 ? 4 : 2);
  constexpr int VS = vt_stride_bytes(VF32);

  auto stage_v = [&](int it) {
    if (VF32) {
      // items: (c, slot, 4-feature group)
      const int groups = C::kDP / 4;
      for (int item = tid; item < kCH * 32 * groups; item += C::kThreads) {
        const int g = item % groups;
        const int slot = (item / groups) & 31;
        const int c = item / (groups * 32);
        const int gc = it * kCH + c;
        const int key = (slot >> 4) * Hh + 16 * gc + (slot & 15);
        const bool kv = (gc < nchunk) && key < kend;
        const float* src = reinterpret_cast<const float*>(vsrc) + static_cast<int64_t>(key) * d;
        float f[4];
        if (kv && (d & 3) == 0 && 4 * g + 4 <= d) {
          const float4 t4 = *reinterpret_cast<const float4*>(src + 4 * g);
          f[0] = t4.x; f[1] = t4.y; f[2] = t4.z; f[3] = t4.w;
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) f[k] = (kv && 4 * g + k < d) ? src[4 * g + k] : 0.0f;
        }
        unsigned char* dst = region + c * C::kDP * VS + slot * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) *reinterpret_cast<float*>(dst + (4 * g + k) * VS) = f[k];
      }
    } else {
      // items: (c, slot pair, 8-feature group)
      const int groups = C::kDP / 8;
      for (int item = tid; item < kCH * 16 * groups; item += C::kThreads) {
        const int g = item % groups;
        const int sp = (item / groups) & 15;
        const int c = item / (groups * 16);
        const int gc = it * kCH + c;
        const int slot = 2 * sp;
        const int key = (slot >> 4) * Hh + 16 * gc + (slot & 15);
        uint32_t h0[4], h1[4];
        const uint16_t* src = reinterpret_cast<const uint16_t*>(vsrc);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          uint32_t* h = kk ? h1 : h0;
          const bool kv = (gc < nchunk) && (key + kk) < kend;
          const uint16_t* row = src + static_cast<int64_t>(key + kk) * d;
          if (kv && (d & 7) == 0 && 8 * g + 8 <= d) {
            const u32x4 t = *reinterpret_cast<const u32x4*>(row + 8 * g);
            h[0] = t[0]; h[1] = t[1]; h[2] = t[2]; h[3] = t[3];
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const uint32_t lo = (kv && 8 * g + 2 * k < d) ? row[8 * g + 2 * k] : 0u;
              const uint32_t hi = (kv && 8 * g + 2 * k + 1 < d) ? row[8 * g + 2 * k + 1] : 0u;
              h[k] = lo | (hi << 16);
            }
          }
        }
        unsigned char* dst = region + c * C::kDP * VS + slot * 2;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // feature 8g+2k: (key, key+1) low halves; feature 8g+2k+1: high halves
          *reinterpret_cast<uint32_t*>(dst + (8 * g + 2 * k) * VS) = (h0[k] & 0xFFFFu) | (h1[k] << 16);
          *reinterpret_cast<uint32_t*>(dst + (8 * g + 2 * k + 1) * VS) = (h0[k] >> 16) | (h1[k] & 0xFFFF0000u);
        }
      }
    }
  };

  for (int it = 0; it < niter; ++it) {
    __syncthreads();
    stage_k(it);
    stage_v(it);
    __syncthreads();
    for (int c = 0; c < kCH; ++c) {
      const int gc = it * kCH + c;
      if (gc >= nchunk) break;
      if (16 * gc >= wlim) break;
      const v16i s = logits_tile(c);
      const int L = lim - (half * Hh + 16 * gc);
      const bool full = __all(L >= 16);
      uint32_t e[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool valid = full || i < L;
        const bool eq = valid && (s[i] == sT);
        const bool keep = (valid && s[i] > sT) || (eq && quota > 0);
        quota -= eq ? 1 : 0;
        const int li = keep ? (((lut_off - s[i]) >> 1)) : kZeroSlot;
        e[i] = wlut[li];
      }
      const unsigned char* vbase = region + c * C::kDP * VS;
      if (VF32) {
#pragma unroll
        for (int t = 0; t < W; ++t) {
          const unsigned char* vrow = vbase + (32 * t + ql) * VS + 64 * half;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float av = *reinterpret_cast<const float*>(vrow + 4 * i);
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, u2f(e[i]), acc[t], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int ab = 0; ab < 2; ++ab) {
          u32x4 ph, pl;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t e0 = e[8 * ab + 2 * k], e1 = e[8 * ab + 2 * k + 1];
            ph[k] = (e0 & 0xFFFFu) | (e1 << 16);
            pl[k] = (e0 >> 16) | (e1 & 0xFFFF0000u);
          }
          const v8bf bh8 = __builtin_bit_cast(v8bf, ph);
          const v8bf bl8 = __builtin_bit_cast(v8bf, pl);
#pragma unroll
          for (int t = 0; t < W; ++t) {
            const u32x4 vv = *reinterpret_cast<const u32x4*>(vbase + (32 * t + ql) * VS + 32 * half + 16 * ab);
            const v8bf av = __builtin_bit_cast(v8bf, vv);
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bh8, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bl8, acc[t], 0, 0, 0);
          }
        }
      }
    }
  }

  // =========================================================== epilogue
  if (!qvalid) return;
  float* orow = a.out + (bh * n + i_row) * static_cast<int64_t>(d);
#pragma unroll
  for (int t = 0; t < W; ++t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f0 = 32 * t + 8 * j + 4 * half;
      const float o0 = acc[t][4 * j + 0] * invZ, o1 = acc[t][4 * j + 1] * invZ;
      const float o2 = acc[t][4 * j + 2] * invZ, o3 = acc[t][4 * j + 3] * invZ;
      if ((d & 3) == 0 && f0 + 4 <= d) {
        *reinterpret_cast<float4*>(orow + f0) = make_float4(o0, o1, o2, o3);
      } else {
        if (f0 + 0 < d) orow[f0 + 0] = o0;
        if (f0 + 1 < d) orow[f0 + 1] = o1;
        if (f0 + 2 < d) orow[f0 + 2] = o2;
        if (f0 + 3 < d) orow[f0 + 3] = o3;
      }
    }
  }
}

template <int W, bool VF32, int MODE>
had_status launch_one(const AttnArgs& a, hipStream_t st) {
  using C = Cfg<W>;
  const int qrows = (MODE == 2) ? a.row_count : a.n;
  const int64_t ntq = (qrows + C::kQB - 1) / C::kQB;
  const int64_t blocks = ntq * a.bh_count;
  if (blocks <= 0) return HAD_OK;
  if (blocks > 0x7FFFFFFF) return fail(HAD_ERR_UNSUPPORTED, "grid too large");
  const size_t lds = lds_bytes<W, VF32>(a.d);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&had_attn_kernel<W, VF32, MODE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) {
      set_error("hipFuncSetAttribute(%zu B LDS) failed: %s", lds, hipGetErrorString(e));
      return HAD_ERR_HIP;
    }
  }
  had_attn_kernel<W, VF32, MODE><<<static_cast<unsigned>(blocks), C::kThreads, lds, st>>>(a);
  return check_launch(MODE == 0 ? "had_attention" : (MODE == 1 ? "had_select" : "had_logits"));
}

template <int W>
had_status launch_w(AttnMode mode, const AttnArgs& a, hipStream_t st) {
  switch (mode) {
    case AttnMode::Attend:
      return a.v_dtype == HAD_F32 ? launch_one<W, true, 0>(a, st) : launch_one<W, false, 0>(a, st);
    case AttnMode::Select:
      return launch_one<W, false, 1>(a, st);
    case AttnMode::Logits:
      return launch_one<W, false, 2>(a, st);
  }
  return fail(HAD_ERR_INVALID_ARG, "unknown mode");
}

}  // namespace

had_status launch_attention_family(AttnMode mode, const AttnArgs& a, hipStream_t st) {
  switch (words_per_row(a.d)) {
    case 1: return launch_w<1>(mode, a, st);
    case 2: return launch_w<2>(mode, a, st);
    case 3: return launch_w<3>(mode, a, st);
    case 4: return launch_w<4>(mode, a, st);
    case 5: return launch_w<5>(mode, a, st);
    case 6: return launch_w<6>(mode, a, st);
    case 7: return launch_w<7>(mode, a, st);
    case 8: return launch_w<8>(mode, a, st);
  }
  return fail(HAD_ERR_UNSUPPORTED, "dim outside [1, 256]");
}

}  // namespace had
