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
//  * Logits on the int8 matrix cores.  v_mfma_i32_32x32x32_i8 computes
//    c + k*u, u = -s, exactly for a tile of 32 keys x 32 queries and 32
//    features: the Q operand holds -k*q as bytes (k = 64 in pass 1, 2 in
//    pass 2; zero in the pad features), the K operand is expanded per wave
//    from the packed key words in LDS through a 256-entry byte table, and the
//    accumulator starts at a per-lane LDS base c.  The result is then directly
//    the LDS address of the element's histogram bin (pass 1) or weight-table
//    entry (pass 2): no address arithmetic per element.
//  * Key order.  The block's visible key range [0, kend) is split at Hh into
//    two halves.  In the output tile the registers i = 0..15 of lane L hold
//    query L%32 and keys half*Hh + 16*chunk + i with half = L/32, so every lane
//    walks its half of the keys in ascending order.  "Lower index wins" among
//    the tied keys then reduces to a per-lane running count.
//  * Selection, pass 1.  Per-wave LDS histogram over the d+1 possible logits:
//    dword [bin][query] holds the half-0 count in its low and the half-1
//    count in its high 16 bits (ds_add_u32 of 1 or 1<<16; the two lane halves
//    run in separate LDS cycles, 32 distinct queries per cycle = 32 banks).
//    A scan per row gives the threshold bin T, the tie quota r split over the
//    halves, h_min and the softmax denominator Z (from counts, without V).
//  * Pass 2.  The logits are recomputed on the matrix cores (cheaper than
//    storing them), each element is kept or dropped with one compare of a
//    composite key (its table address shifted left by 15 plus the running
//    tie count), its weight exp(-2*scale*(h - h_min)) is read from an LDS
//    table as a pair of bf16 terms (hi + lo, relative error < 2^-15), and
//    out^T = V^T P^T runs on v_mfma_f32_32x32x16_bf16 (two products, hi and
//    lo) with V staged transposed in LDS.  fp32 V uses v_mfma_f32_32x32x2_f32
//    with fp32 weights.  Dense-masked products on the matrix cores beat a
//    per-row gather of the N kept V rows: a gather reads 2*d bytes of on-chip
//    bandwidth per kept pair, the tile product reuses every staged V row for
//    32 query rows.
//  * Staging.  Key words (and, in pass 2, V rows) of the next key group are
//    copied into the other LDS buffer with asynchronous global-to-LDS loads
//    while the current group is computed: one barrier per key group.  fp32 V
//    and feature counts that are not a multiple of 32 go through registers
//    and are stored transposed.  Groups are large (pass 1: 4 KB of key words;
//    pass 2: about 16 KB of V) so that the compute of one group hides the load
//    latency of the next.
#include <atomic>

#include "had_internal.h"

namespace had {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Build option: the logit tiles from XOR + popcount on the vector ALU instead
// of the int8 matrix cores (the same tile values, so the same results; the
// K-only sweeps then take their plain loop).  It builds libhad_popcount.so,
// the comparison that keeps the matrix-core stage in libhad.so.
#ifndef HAD_LOGITS_POPCOUNT
#define HAD_LOGITS_POPCOUNT 0
#endif
constexpr bool kPopcountLogits = HAD_LOGITS_POPCOUNT != 0;

// Build option: the attend launch takes the float32 Q rows and forms their
// sign words itself (Q's pack fused into the attention launch), writing the
// words and per-wave sigma partials on the side.  It builds
// libhad_fusedq.so, the measurement of that fusion against had_forward's
// separate pack launch.
#ifndef HAD_FUSED_QPACK
#define HAD_FUSED_QPACK 0
#endif
constexpr bool kFusedQ = HAD_FUSED_QPACK != 0;

// weight table: d+1 weights, then a zero slot in the last bank of its
// 64-dword row, away from the low entries every row uses
constexpr int kLutEntries = 320;
constexpr int kZeroSlot = 319;
constexpr int kByteLutOff = 0;          // 256 x 8 B: byte -> 8 int8 of +-1
constexpr int kWLutOff = 2048;          // kLutEntries x 4 B
constexpr int kKbOff = kWLutOff + 4 * kLutEntries;

__host__ __device__ constexpr int waves_for(int W) { return W <= 4 ? 4 : 2; }
__host__ __device__ constexpr int threads_for(int W) { return 64 * waves_for(W); }
// Register budget of the bf16 attention kernel with directly copied V
// tiles: at d <= 64 keep 3 waves per SIMD (<= 168 VGPRs); otherwise 2.
__host__ __device__ constexpr int min_waves_for(int W, bool vf32, int mode, bool vdirect) {
  return (W <= 2 && !vf32 && mode == 0 && vdirect) ? 3 : 2;
}
__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int W, bool VF32, bool VDIRECT>
struct Cfg {
  static constexpr int kWaves = waves_for(W);
  static constexpr int kThreads = threads_for(W);
  static constexpr int kQB = 32 * kWaves;  // query rows per block
  static constexpr int kDP = 32 * W;       // padded feature count
  // 16-key chunks per half in one key group: K-only loops (4 KB of key
  // words; fewer groups mean fewer barriers and pipeline refills) and the
  // attend loop (V tile of about 16 KB)
  static constexpr int kCH1 = 32 / W;
  static constexpr int kCH2 = VF32 ? (W <= 2 ? 2 : 1) : (W <= 2 ? 4 : (W <= 4 ? 2 : 1));
  static constexpr int kKb1 = kCH1 * 32 * W * 4;  // bytes of key words per group
  static constexpr int kKb2 = kCH2 * 32 * W * 4;
  static constexpr int kKbBuf = cmax(kKb1, kKb2);
  static constexpr int kVS = VF32 ? 144 : 80;     // bytes per staged feature row
  // V tile: transposed [feature][slot] rows of kVS bytes, or (VDIRECT) the
  // row-major [slot][feature] rows copied straight from global memory
  static constexpr int kVBuf = VDIRECT ? kCH2 * 32 * 2 * kDP : kCH2 * kDP * kVS;
  static constexpr int kHist = kWaves * (kDP + 1) * 32 * 4;
  static constexpr int kRegionOff = kKbOff + 2 * kKbBuf;
  static constexpr int kLdsBytes = kRegionOff + cmax(kHist, 2 * kVBuf);
  // 16-byte pieces of a row-major V row, and the piece swizzle that makes the
  // transposed operand reads bank-conflict free (power-of-two rows only)
  static constexpr int kPieces = kDP / 8;
  static constexpr int kSwzMask = ((kPieces & (kPieces - 1)) == 0) ? (kPieces - 1) & 6 : 0;
};

__device__ inline uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ inline float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t u = f2u(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ inline float bf16_to_f(uint32_t b) { return u2f(b << 16); }

// 4 sign bits -> 4 int8 lanes of +k (bit 0) / -k (bit 1); pos is the byte
// of +k and flip = byte(+k) ^ byte(-k).
__device__ inline uint32_t expand_nibble_k(uint32_t nib, uint32_t pos, uint32_t flip) {
  const uint32_t y = (nib * 0x00204081u) & 0x01010101u;  // bit k -> byte k
  return (y * flip) ^ (pos * 0x01010101u);
}
__device__ inline uint32_t expand_nibble(uint32_t nib) { return expand_nibble_k(nib, 0x01u, 0xFEu); }

// Byte mask keeping the features [base, base+4) that are < d.
__device__ inline uint32_t pad_mask4(int base, int d) {
  const int valid = d - base;
  if (valid >= 4) return 0xFFFFFFFFu;
  if (valid <= 0) return 0u;
  return (1u << (8 * valid)) - 1u;
}

// LDS byte address (address space 3) of a location in the kernel's LDS array.
typedef __attribute__((address_space(3))) unsigned char lds_byte;
typedef __attribute__((address_space(3))) const uint32_t lds_cu32;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) void lds_void;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
__device__ inline uint32_t lds_addr(const unsigned char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_byte*)p));
}
__device__ inline uint32_t lds_load_u32(uint32_t addr) {
  return *(lds_cu32*)(static_cast<uintptr_t>(addr));
}
// Issue priority of the calling wave (0..3, higher issues first).  When the
// whole grid is resident at once, the work-groups that share a CU start
// together and have equal work, but the instruction arbiter favours the
// oldest waves: without help the first work-group races ahead and the last
// one finishes alone, with a third of the waves to hide its latencies.
// Lowering a wave's priority as it progresses (3 in pass 1, then 2, 1 and,
// for the last key group only, 0) lets the ones behind issue first; within
// one level the oldest still goes first, so the last level is kept short.
__device__ inline void set_priority(int p) {
  switch (p) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// Keeps a per-lane value in a VGPR as computed (stops re-association that
// would split an LDS base back out of it).
__device__ inline uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int W, bool VF32, int MODE, bool VDIRECT>
__global__ __launch_bounds__(threads_for(W))
__attribute__((amdgpu_waves_per_eu(min_waves_for(W, VF32, MODE, VDIRECT))))
void had_attn_kernel(AttnArgs a) {
  using C = Cfg<W, VF32, VDIRECT>;
  constexpr int VS = C::kVS;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::kLdsBytes];
  const uint2* byte_lut = reinterpret_cast<const uint2*>(lds + kByteLutOff);
  uint32_t* wlut = reinterpret_cast<uint32_t*>(lds + kWLutOff);
  unsigned char* region = lds + C::kRegionOff;  // histograms (pass 1) | V tiles (pass 2)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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
  // keys j < lim are visible to this lane's query row
  const int lim = !qvalid ? 0 : (causal ? min(i_row + 1, n) : n);
  const int wave_q0 = q0 + wid * 32;
  const int wlim = (wave_q0 >= qend) ? 0 : (causal ? min(n, wave_q0 + 32) : n);
  const int wchunks = min(nchunk, (wlim + 15) / 16);  // chunks with keys this wave sees

  // ---- key words: kb[c][m][w], m = MFMA row of the logit tile.  Row m holds
  // key (m>>2 & 1)*Hh + 16*gc + 4*(m>>3) + (m&3), i.e. register i of lane L
  // gets key half*Hh + 16*gc + i.  Pad features need no masking: the Q
  // operand is zero there.
  const uint32_t* kbg = a.kbits + bh * static_cast<int64_t>(n) * W;
  auto key_of = [&](int gc, int m) { return ((m >> 2) & 1) * Hh + 16 * gc + 4 * (m >> 3) + (m & 3); };
  // Copies the key words of chunks [g0, g0 + ch) straight into buffer buf
  // (global_load_lds, 4 bytes per lane, lane-ordered); keys outside the
  // visible range load a valid row (their logits are masked).  The per-lane
  // part of each copy address is fixed; only the group base 16*g0 moves, and
  // offsets stay 32-bit within the slice.
  auto k_issue = [&](int g0, auto ch_c, int buf) {
    constexpr int kItems = decltype(ch_c)::value * 32 * W;
    constexpr int kJ = (kItems + 64 * C::kWaves - 1) / (64 * C::kWaves);
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) {
      const int j = wid + jj * C::kWaves;
      const int item = j * 64 + lane;
      if (item < kItems) {
        const int w = item % W;
        const int m = (item / W) & 31;
        const int c = item / (W * 32);
        // keys past the visible range (never used) load a valid row
        const int key = min(key_of(c, m) + 16 * g0, kend - 1);
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const uint32_t*>(reinterpret_cast<const unsigned char*>(kbg) +
                                              static_cast<uint32_t>(4 * (key * W + w))),
            (lds_void*)(lds + kKbOff + buf * C::kKbBuf + j * 256), 4, 0, 0);
      }
    }
  };
  // all of this thread's copies have landed; then the block barrier
  auto copies_done = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // the first key group of the first sweep is in flight during the set-up
  k_issue(0, std::integral_constant<int, C::kCH1>{}, 0);

  // ---- sigma of the fused forward call: wave 0 of the last block (the
  // lightest one when causal) reduces the pack partials before its own work
  if (MODE == 0 && wid == 0 && blockIdx.x == gridDim.x - 1) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (a.sigma_out[t] != nullptr)
        sigma_from_partials(a.sigma_partials[t], a.sigma_nparts, a.sigma_count, a.sigma_out[t]);
  }

  // ---- constant tables
  for (int t = tid; t < 256; t += C::kThreads)
    reinterpret_cast<uint2*>(lds + kByteLutOff)[t] =
        make_uint2(expand_nibble(t & 15u), expand_nibble(t >> 4));
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

  // ---- Q operand: -k*q as bytes, features 32w + 16*half + [0,16); pad = 0
  v4i qx[W];
  uint32_t qwords[W];
  // (the fused form is taken only by a forward call, which passes the float32
  // rows; had_attention in the same build passes sign words as usual)
  if (kFusedQ && MODE == 0 && a.qf != nullptr) {
    // float32 Q rows: this lane forms the 16 sign bits of each word that its
    // half of the Q operand uses (features 32w + 16*half + [0, 16)); the two
    // halves of a row swap theirs so that half 0 stores the row's words; the
    // lane's float64 sums of the elements minus the tensor's first element
    // (0 if not finite), as in had_pack, give one sigma partial pair per wave
    const float* xr = a.qf + (bh * n + (qvalid ? i_row : 0)) * static_cast<int64_t>(d);
    const float x0 = a.qf[0];
    const float csh = __builtin_isfinite(x0) ? x0 : 0.0f;
    double s1 = 0.0, s2 = 0.0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const int f0 = 32 * w + 16 * half;
      float x[16];
      if (a.qf_vec) {
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          const float4 t = qvalid ? *reinterpret_cast<const float4*>(xr + f0 + j) : make_float4(0.f, 0.f, 0.f, 0.f);
          x[j] = t.x; x[j + 1] = t.y; x[j + 2] = t.z; x[j + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = (qvalid && f0 + j < d) ? xr[f0 + j] : 0.0f;
      }
      uint32_t b16 = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const bool in = qvalid && f0 + j < d;
        b16 |= static_cast<uint32_t>(in && x[j] < 0.0f) << j;
        const double y = in ? static_cast<double>(x[j] - csh) : 0.0;
        s1 += y;
        s2 = fma(y, y, s2);
      }
      qwords[w] = ~(b16 << (16 * half));  // complement: the product is -s (only this half's bits are used)
      const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(b16), 32, 64));
      if (qvalid && half == 0) a.qbits_out[(bh * n + i_row) * W + w] = b16 | (other << 16);
    }
    s1 = wave_sum_f64(s1);
    s2 = wave_sum_f64(s2);
    if (lane == 63) {
      if (a.qpartials != nullptr) {
        double* pp = a.qpartials + 2 * (static_cast<int64_t>(blockIdx.x) * C::kWaves + wid);
        pp[0] = s1;
        pp[1] = s2;
      }
      if (s2 != s2 && a.dev_status != nullptr) atomicOr(a.dev_status, HAD_DEV_NAN_INPUT);
    }
  } else {
    const uint32_t* qrow = a.qbits + (bh * n + (qvalid ? i_row : 0)) * W;
#pragma unroll
    for (int w = 0; w < W; ++w) qwords[w] = qvalid ? ~qrow[w] : ~0u;  // complement: the product is -s
  }
  int kmag = 0;  // k of the tile entries cin + k*u (the popcount build uses it)
  auto make_q = [&](uint32_t pos, uint32_t flip) {
    kmag = static_cast<int>(pos);
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const uint32_t b16 = (qwords[w] >> (16 * half)) & 0xFFFFu;
      const int fbase = 32 * w + 16 * half;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        qx[w][k] = static_cast<int>(expand_nibble_k((b16 >> (4 * k)) & 15u, pos, flip) &
                                    pad_mask4(fbase + 4 * k, d));
    }
  };

  // cin + k*u, u = -logit, for (query ql, key half*Hh + 16*gc + i),
  // i = 0..15, chunk c of the key-word buffer buf (k set by make_q), in
  // three steps that a caller can spread out to hide their LDS latency:
  // the key words, their +-1 bytes (table reads), the products.
  auto k_words = [&](int buf, int c, uint32_t (&words)[W]) {
    const uint32_t* krow = reinterpret_cast<const uint32_t*>(lds + kKbOff + buf * C::kKbBuf) + (c * 32 + ql) * W;
#pragma unroll
    for (int w = 0; w < W; ++w) words[w] = krow[w];
  };
  auto k_expand = [&](const uint32_t (&words)[W], v4i (&kv)[W]) {
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const uint32_t b16 = words[w] >> (16 * half);
      const uint2 lo = byte_lut[b16 & 0xFFu];
      const uint2 hi = byte_lut[(b16 >> 8) & 0xFFu];
      kv[w] = v4i{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(hi.x), static_cast<int>(hi.y)};
    }
  };
  auto k_product = [&](const v4i (&kv)[W], uint32_t cin) {
    v16i acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = static_cast<int>(cin);
#pragma unroll
    for (int w = 0; w < W; ++w) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kv[w], qx[w], acc, 0, 0, 0);
    return acc;
  };
  auto logits_tile = [&](int buf, int c, uint32_t cin) {
    if constexpr (kPopcountLogits) {
      // u = 2h - d with h = sum over words of popcount(q XOR k) (pad bits are
      // 0 in both), for the keys of this lane's registers (MFMA rows m)
      const uint32_t* kb = reinterpret_cast<const uint32_t*>(lds + kKbOff + buf * C::kKbBuf) + c * 32 * W;
      const uint32_t base = cin - static_cast<uint32_t>(kmag * d);
      const uint32_t k2 = static_cast<uint32_t>(2 * kmag);
      v16i t;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = ((i >> 2) << 3) | (half << 2) | (i & 3);
        uint32_t h = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) h = __builtin_popcount(~qwords[w] ^ kb[m * W + w]) + h;
        t[i] = static_cast<int>(base + k2 * h);
      }
      return t;
    } else {
      uint32_t words[W];
      v4i kv[W];
      k_words(buf, c, words);
      k_expand(words, kv);
      return k_product(kv, cin);
    }
  };

  // K-only sweep over all chunks this wave sees, kCH1 chunks per group;
  // body(u, gc, full) runs per chunk; full (a compile-time tag) says that
  // every lane of the wave sees all 16 keys of the chunk.
  // first_issued: group 0 was copied at kernel entry.
  auto k_sweep = [&](uint32_t cin, bool first_issued, auto&& body) {
    const int ngroups = (nchunk + C::kCH1 - 1) / C::kCH1;
    if (!first_issued) {
      __syncthreads();  // previous users of the key buffers are done
      k_issue(0, std::integral_constant<int, C::kCH1>{}, 0);
    }
    copies_done();
    for (int gi = 0; gi < ngroups; ++gi) {
      const int buf = gi & 1;
      if (a.balance && gi == 0) set_priority(3);
      if (gi + 1 < ngroups) k_issue((gi + 1) * C::kCH1, std::integral_constant<int, C::kCH1>{}, buf ^ 1);
      const int g0 = gi * C::kCH1;
      const int cend = min(C::kCH1, wchunks - g0);
      // every lane sees every key of the group: keys up to half*Hh + 16*(g0 + kCH1)
      const bool whole = !kPopcountLogits && cend == C::kCH1 && __all(lim >= half * Hh + 16 * (g0 + C::kCH1));
      if (whole) {
        // A full group, software-pipelined and straight-line: step c takes
        // the products of chunk c, expands the key bytes of chunk c + 2,
        // reads the key words of chunk c + 3 and hands chunk c - 1 to the
        // body.  A product's operands were read a whole step (and one
        // body's worth of LDS atomics) before it, and with no branch in
        // between the compiler's waits stop at exactly those reads.
        constexpr int K = C::kCH1;
        uint32_t kw[W];
        v4i kv0[W], kv1[W];
        v16i ta, tb;
        auto step = [&](v16i& cur, const v16i& prev, v4i (&kv)[W], int c) {
          cur = k_product(kv, cin);
          if (c + 2 < K) k_expand(kw, kv);
          if (c + 3 < K) k_words(buf, c + 3, kw);
          if (c > 0) body(prev, g0 + c - 1, std::true_type{});
        };
        k_words(buf, 0, kw);
        k_expand(kw, kv0);
        if (K > 1) {
          k_words(buf, 1, kw);
          k_expand(kw, kv1);
        }
        if (K > 2) k_words(buf, 2, kw);
#pragma unroll
        for (int c = 0; c < K; c += 2) {
          step(ta, tb, kv0, c);
          if (c + 1 < K) step(tb, ta, kv1, c + 1);
        }
        body((K & 1) ? ta : tb, g0 + K - 1, std::true_type{});
      } else if (cend > 0) {
        v16i u_next = logits_tile(buf, 0, cin);
        for (int c = 0; c < cend; ++c) {
          const v16i u = u_next;
          if (c + 1 < cend) u_next = logits_tile(buf, c + 1, cin);
          body(u, g0 + c, std::false_type{});
        }
      }
      copies_done();
    }
  };

  // =========================================================== logits export
  if (MODE == 2) {
    int16_t* dst = a.logits + (bh_local * a.row_count + (qvalid ? i_row - a.row_begin : 0)) * static_cast<int64_t>(n);
    make_q(0x01u, 0xFEu);  // +-1: the tile holds u itself
    k_sweep(0u, true, [&](const v16i& u, int gc, auto) {
      if (!qvalid) return;
      const int kbase = half * Hh + 16 * gc;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kbase + i < lim) dst[kbase + i] = static_cast<int16_t>(-u[i]);
    });
    return;
  }

  // =========================================================== pass 1: histogram
  {
    uint32_t* hist = reinterpret_cast<uint32_t*>(region) + wid * (d + 1) * 32;
    for (int t = lane; t < (d + 1) * 32; t += 64) hist[t] = 0u;
  }
  const uint32_t addend = half ? 0x10000u : 1u;
  // LDS address of bin (d + u)/2 for this lane's query: hb + 64*u, which is
  // what the tile holds with k = 64 and cin = hb
  const uint32_t hb = lds_addr(region + (wid * (d + 1) * 32 + ql) * 4 + 64 * d);
  make_q(0x40u, 0x80u);  // +-64
  k_sweep(hb, true, [&](const v16i& t, int gc, auto full) {
    if constexpr (decltype(full)::value) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __atomic_fetch_add((lds_u32*)(static_cast<uintptr_t>(static_cast<uint32_t>(t[i]))), addend, __ATOMIC_RELAXED);
    } else {
      // element i visible iff i < L; hidden ones add 0 (their tile entry is
      // a valid bin address)
      const int L = lim - (half * Hh + 16 * gc);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __atomic_fetch_add((lds_u32*)(static_cast<uintptr_t>(static_cast<uint32_t>(t[i]))), i < L ? addend : 0u,
                           __ATOMIC_RELAXED);
    }
  });

  // the key buffers are free again (the sweep ended with a barrier): the
  // first key group of pass 2 is copied while the statistics are computed
  if (MODE == 0) k_issue(0, std::integral_constant<int, C::kCH2>{}, 0);

  if (MODE == 3) {
    // ===================================================== top-N mass export
    // Smallest N whose N largest softmax weights reach mass * Z: the keys of
    // a histogram bin share one weight w_h = exp(-2*scale*(h - h_min)), so
    // the largest weights are whole bins from h_min up, then ceil(rest / w_T)
    // keys of the bin T where the running sum crosses (float64 throughout).
    if (qvalid && half == 0) {
      const uint32_t* hq3 = reinterpret_cast<const uint32_t*>(region) + wid * (d + 1) * 32 + ql;
      int hmin3 = -1;
      double Z = 0.0;
      for (int b = 0; b <= d; ++b) {
        const uint32_t x = hq3[b * 32];
        const int cnt = static_cast<int>(x & 0xFFFFu) + static_cast<int>(x >> 16);
        if (cnt > 0 && hmin3 < 0) hmin3 = b;
        if (cnt > 0) Z += cnt * exp(-2.0 * static_cast<double>(a.scale) * (b - hmin3));
      }
      int N = lim;  // mass >= 1, or a rounding shortfall: every visible key
      if (a.mass < 1.0) {
        const double target = a.mass * Z;
        double M = 0.0;
        int before = 0;
        for (int b = hmin3; b <= d; ++b) {
          const uint32_t x = hq3[b * 32];
          const int cnt = static_cast<int>(x & 0xFFFFu) + static_cast<int>(x >> 16);
          if (cnt == 0) continue;
          const double w = exp(-2.0 * static_cast<double>(a.scale) * (b - hmin3));
          if (M + cnt * w >= target) {
            int k = static_cast<int>(ceil((target - M) / w));
            k = k < 1 ? 1 : (k > cnt ? cnt : k);
            N = before + k;
            break;
          }
          M += cnt * w;
          before += cnt;
        }
      }
      a.nmass[bh_local * n + i_row] = N;
    }
    return;
  }

  // =========================================================== per-row statistics
  const int Ni = qvalid ? min(a.topn, lim) : 0;
  const uint32_t* hq = reinterpret_cast<const uint32_t*>(region) + wid * (d + 1) * 32 + ql;
  int T, hmin, below0, ties0, below;
  {
    // Scan the bins upward, 8 independent LDS reads at a time, keeping the
    // running counts packed as the histogram stores them (half 0 | half 1
    // << 16; each stays below 2^16): one add per bin, the total by a dot
    // product with (1, 1).  The running total never decreases, so T is the
    // number of bins whose running total is still below Ni, h_min the number
    // whose running total is 0, and the counts below T are the running
    // counts at the last bin below Ni.  The wave stops once every lane has
    // passed its Ni (the visible count is >= Ni, so every lane does).
    typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
    const v2u16 ones = {1, 1};
    const uint32_t ni = static_cast<uint32_t>(Ni);
    uint32_t cumx = 0, cumx_lt = 0;
    int nlt = 0, nzero = 0;
    for (int b0 = 0; b0 <= d; b0 += 8) {
      uint32_t x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = (b0 + k <= d) ? hq[(b0 + k) * 32] : 0u;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        cumx += x[k];
        const uint32_t tot = __builtin_amdgcn_udot2(__builtin_bit_cast(v2u16, cumx), ones, 0u, false);
        const bool lt = tot < ni;
        nlt += lt ? 1 : 0;
        cumx_lt = lt ? cumx : cumx_lt;
        nzero += tot == 0u ? 1 : 0;
      }
      if (__all(__builtin_amdgcn_udot2(__builtin_bit_cast(v2u16, cumx), ones, 0u, false) >= ni)) break;
    }
    T = min(nlt, d);
    hmin = cumx == 0u ? 0 : nzero;  // an empty histogram (no visible key) keeps 0
    below0 = static_cast<int>(cumx_lt & 0xFFFFu);
    below = below0 + static_cast<int>(cumx_lt >> 16);
    ties0 = static_cast<int>(hq[T * 32] & 0xFFFFu);
  }
  const int r_tie = Ni - below;
  const int quota0 = min(r_tie, ties0);
  const int quota = half ? (r_tie - quota0) : quota0;
  const int uT = (Ni > 0) ? 2 * T - d : -(d + 2);  // rows with nothing to keep never match
  // Selection works on au = lutc + 2u, the weight-table address of the
  // element (a pass-2 tile with k = 2 and cin = lutc; lutc is set below).
  // Element i of this lane (ascending keys) is kept iff u_i < uT, or
  // u_i == uT and fewer than `quota` ties precede it here, i.e. iff
  //   (au_i - auT) * 2^15 + ties_seen - quota < 0,
  // evaluated as D = (au_i << 15) + sp with sp = ties_seen - quota - (auT << 15)
  // in 32-bit wrap-around arithmetic (au < 2^12, and ties_seen and quota stay
  // below 2^15 + 16 because a half holds at most 32768 + 15 keys).
  const uint32_t lutc = opaque(lds_addr(lds + kWLutOff + 2 * d - 4 * hmin));
  const uint32_t auT = lutc + 2u * static_cast<uint32_t>(uT);
  uint32_t sp = 0u - static_cast<uint32_t>(quota) - (auT << 15);

  if (MODE == 4) {
    // ===================================================== row statistics export
    // For a backward pass that visits the keys in another order: Z in float64
    // from the histogram with float32 weights exp(-2*scale*t), and the index
    // of the last kept key at the threshold.  The kept keys at the threshold
    // are the first r_tie of them in key order, so a key j with logit at the
    // threshold is kept exactly when j <= that index; it is found by walking
    // each half's keys in order as the selection export does (half 1's keys
    // all follow half 0's).
    double z = 0.0;
    if (Ni > 0) {
      for (int b = hmin; b <= T; ++b) {
        const uint32_t x = hq[b * 32];
        const int cnt = b < T ? static_cast<int>(x & 0xFFFFu) + static_cast<int>(x >> 16) : r_tie;
        z += static_cast<double>(cnt) * static_cast<double>(expf(-2.0f * a.scale * static_cast<float>(b - hmin)));
      }
    }
    // Only the visible keys at the threshold matter here: such a key is kept
    // while fewer than this half's quota of them precede it.
    int last_tie = -1;
    int ties = 0;
    make_q(0x02u, 0xFCu);  // +-2
    k_sweep(lutc, false, [&](const v16i& t, int gc, auto full) {
      const int kbase = half * Hh + 16 * gc;
      const int L = lim - kbase;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool tie = (decltype(full)::value || i < L) && static_cast<uint32_t>(t[i]) == auT;
        last_tie = (tie && ties < quota) ? kbase + i : last_tie;
        ties += tie ? 1 : 0;
      }
    });
    last_tie = max(last_tie, __shfl_xor(last_tie, 32, 64));  // lanes L and L ^ 32 share a row
    if (qvalid && half == 0) {
      int32_t* dst = a.rowstats + (bh_local * n + i_row) * static_cast<int64_t>(4);
      *reinterpret_cast<int4*>(dst) = make_int4(T, last_tie, hmin, __builtin_bit_cast(int32_t, static_cast<float>(z)));
    }
    return;
  }

  if (MODE == 1) {
    // ======================================================= selection export
    int pos = half ? (below0 + quota0) : 0;
    int32_t* dst = a.idx + (bh_local * n + (qvalid ? i_row : 0)) * static_cast<int64_t>(a.topn);
    make_q(0x02u, 0xFCu);  // +-2
    k_sweep(lutc, false, [&](const v16i& t, int gc, auto) {
      const int kbase = half * Hh + 16 * gc;
      const int L = lim - kbase;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t au = static_cast<uint32_t>(t[i]);
        const bool keep = i < L && static_cast<int32_t>((au << 15) + sp) < 0;
        sp += (au == auT) ? 1u : 0u;
        if (keep && pos < a.topn) dst[pos++] = kbase + i;
      }
    });
    if (qvalid && half == 0)
      for (int p = Ni; p < a.topn; ++p) dst[p] = -1;
    return;
  }

  // =========================================================== pass 2: attend
  float Z = 0.0f;
  if (Ni > 0) {
    for (int b0 = hmin; b0 < T; b0 += 8) {
      uint32_t x[8], e[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool in = b0 + k < T;
        x[k] = in ? hq[(b0 + k) * 32] : 0u;
        e[k] = in ? wlut[b0 + k - hmin] : 0u;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int cnt = static_cast<int>(x[k] & 0xFFFFu) + static_cast<int>(x[k] >> 16);
        const float w = VF32 ? u2f(e[k]) : bf16_to_f(e[k] & 0xFFFFu) + bf16_to_f(e[k] >> 16);
        Z += static_cast<float>(cnt) * w;
      }
    }
    const uint32_t e = wlut[T - hmin];
    const float w = VF32 ? u2f(e) : bf16_to_f(e & 0xFFFFu) + bf16_to_f(e >> 16);
    Z += static_cast<float>(r_tie) * w;
  }
  const float invZ = (Z > 0.0f) ? 1.0f / Z : 0.0f;
  // weight-table LDS address of u: wlut + 4*((d + u)/2 - hmin) = lutc + 2u
  const uint32_t zaddr = opaque(lds_addr(lds + kWLutOff + 4 * kZeroSlot));

  v16f acc[W];
#pragma unroll
  for (int t = 0; t < W; ++t) acc[t] = v16f{};

  const unsigned char* vsrc = static_cast<const unsigned char*>(a.v) +
                              bh * static_cast<int64_t>(n) * d * (VF32 ? 4 : 2);

  // ---- V staging, VDIRECT: row-major [slot][feature] bf16 tiles copied by
  // global_load_lds (16 bytes per lane).  Piece pp of row r holds features
  // 8*(pp ^ swz(r)) .. +7, swz(r) = 2*(r & 3) (masked to the row), so that
  // the transposed operand reads below hit 32 distinct banks per 16 lanes.
  // Keys outside the visible range copy key 0 (their weights are zero).
  auto v_issue = [&](int g0, int buf) {
    if constexpr (VDIRECT) {
      constexpr int kInst = C::kCH2 * 32 * C::kPieces / 64;
      constexpr int kJ = (kInst + C::kWaves - 1) / C::kWaves;
#pragma unroll
      for (int jj = 0; jj < kJ; ++jj) {
        const int j = wid + jj * C::kWaves;
        if (j < kInst) {
          const int item = j * 64 + lane;
          const int pp = item % C::kPieces;
          const int r = (item / C::kPieces) & 31;
          const int c = item / (C::kPieces * 32);
          // keys past the visible range (weight 0 or never used) copy a valid row
          const int key = min((r >> 4) * Hh + 16 * c + (r & 15) + 16 * g0, kend - 1);
          const int pc = pp ^ ((2 * (r & 3)) & C::kSwzMask);
          __builtin_amdgcn_global_load_lds(
              reinterpret_cast<const uint16_t*>(reinterpret_cast<const unsigned char*>(vsrc) +
                                                static_cast<uint32_t>(2 * (key * d + 8 * pc))),
              (lds_void*)(region + buf * C::kVBuf + j * 1024), 16, 0, 0);
        }
      }
    }
  };

  // ---- V staging, register path (fp32 V, or d not a multiple of 32):
  // transposed vt[buf][c][feature][slot] with slot = 16*half + key offset.
  // bf16 items: (slot pair sp, 4-feature group g, chunk c), sp fastest: the
  // two g parities of a half-wave land 16 banks apart -> conflict-free writes.
  // fp32 items: (slot, 4-feature group, chunk), slot fastest.
  constexpr int kG = C::kDP / 4;
  constexpr int kVItems = VDIRECT ? 0 : (VF32 ? C::kCH2 * 32 * kG : C::kCH2 * 16 * kG);
  constexpr int kVPT = VDIRECT ? 1 : (kVItems + C::kThreads - 1) / C::kThreads;
  uint32_t vreg[kVPT][4];
  auto v_load = [&](int g0) {
    if constexpr (!VDIRECT) {
#pragma unroll
      for (int j = 0; j < kVPT; ++j) {
        const int item = tid + j * C::kThreads;
        if (VF32) {
          const int slot = item & 31;
          const int g = (item >> 5) % kG;
          const int c = item / (32 * kG);
          const int gc = g0 + c;
          const int key = (slot >> 4) * Hh + 16 * gc + (slot & 15);
          const bool kv = item < kVItems && gc < nchunk && key < kend;
          const float* row = reinterpret_cast<const float*>(vsrc) + static_cast<int64_t>(kv ? key : 0) * d;
          if (kv && (d & 3) == 0 && 4 * g + 4 <= d) {
            const u32x4 t = *reinterpret_cast<const u32x4*>(row + 4 * g);
            vreg[j][0] = t[0]; vreg[j][1] = t[1]; vreg[j][2] = t[2]; vreg[j][3] = t[3];
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) vreg[j][k] = (kv && 4 * g + k < d) ? f2u(row[4 * g + k]) : 0u;
          }
        } else {
          const int sp = item & 15;
          const int g = (item >> 4) % kG;
          const int c = item / (16 * kG);
          const int gc = g0 + c;
          const int key = ((2 * sp) >> 4) * Hh + 16 * gc + ((2 * sp) & 15);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const bool kv = item < kVItems && gc < nchunk && key + kk < kend;
            const uint16_t* row = reinterpret_cast<const uint16_t*>(vsrc) + static_cast<int64_t>(kv ? key + kk : 0) * d;
            if (kv && (d & 3) == 0 && 4 * g + 4 <= d) {
              const uint2 t = *reinterpret_cast<const uint2*>(row + 4 * g);
              vreg[j][2 * kk] = t.x;
              vreg[j][2 * kk + 1] = t.y;
            } else {
              uint32_t f[4];
#pragma unroll
              for (int k = 0; k < 4; ++k) f[k] = (kv && 4 * g + k < d) ? row[4 * g + k] : 0u;
              vreg[j][2 * kk] = f[0] | (f[1] << 16);
              vreg[j][2 * kk + 1] = f[2] | (f[3] << 16);
            }
          }
        }
      }
    }
  };
  auto v_store = [&](int buf) {
    if constexpr (!VDIRECT) {
      unsigned char* vt = region + buf * C::kVBuf;
#pragma unroll
      for (int j = 0; j < kVPT; ++j) {
        const int item = tid + j * C::kThreads;
        if (item >= kVItems) break;
        if (VF32) {
          const int slot = item & 31;
          const int g = (item >> 5) % kG;
          const int c = item / (32 * kG);
          unsigned char* dst = vt + (c * C::kDP + 4 * g) * VS + 4 * slot;
#pragma unroll
          for (int k = 0; k < 4; ++k) *reinterpret_cast<uint32_t*>(dst + k * VS) = vreg[j][k];
        } else {
          const int sp = item & 15;
          const int g = (item >> 4) % kG;
          const int c = item / (16 * kG);
          unsigned char* dst = vt + (c * C::kDP + 4 * g) * VS + 4 * sp;
          const uint32_t a0 = vreg[j][0], a1 = vreg[j][1], b0 = vreg[j][2], b1 = vreg[j][3];
          // feature 4g+k: (key, key+1) packed as one dword
          *reinterpret_cast<uint32_t*>(dst + 0 * VS) = __builtin_amdgcn_perm(b0, a0, 0x05040100u);
          *reinterpret_cast<uint32_t*>(dst + 1 * VS) = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
          *reinterpret_cast<uint32_t*>(dst + 2 * VS) = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
          *reinterpret_cast<uint32_t*>(dst + 3 * VS) = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
        }
      }
    }
  };

  // Transposed-read addressing (VDIRECT): within each 16-lane group G, lane
  // 4k+q supplies the 8-byte row piece (slot S + k, features f0 + 4q) and
  // ds_read_b64_tr_b16 returns to lane j the four values (slot S + k,
  // feature f0 + j), k = 0..3.  S = 16*(G>>1) + 8*ab + 4*second_read,
  // f0 = 32*t + 16*(G&1).
  const int trG = lane >> 4, trk = (lane >> 2) & 3, trq = lane & 3;
  const int tr_row = 16 * (trG >> 1) + trk;                 // + 8*ab + 4*second
  const int tr_swz = (2 * trk) & C::kSwzMask;               // slot & 3 == trk
  const int tr_f = 16 * (trG & 1) + 4 * trq;                // + 32*t
  auto v_operand = [&](const unsigned char* vchunk, int t, int ab) {
    const int f = 32 * t + tr_f;
    const int off = (tr_row + 8 * ab) * 2 * C::kDP + (((f >> 3) ^ tr_swz) << 4) + 2 * (f & 7);
    const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vchunk + off));
    const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vchunk + off + 4 * 2 * C::kDP));
    const u32x4 u = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(r0, r0, 0, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_shufflevector(r0, r0, 2, 3)),
                     __builtin_bit_cast(uint32_t, __builtin_shufflevector(r1, r1, 0, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_shufflevector(r1, r1, 2, 3))};
    return __builtin_bit_cast(v8bf, u);
  };

  // out^T += V^T P^T for chunk c of the V tile vt, weights e.
  auto pv_chunk = [&](const unsigned char* vt, int c, const uint32_t* e) {
    if constexpr (VF32) {
      const unsigned char* vbase = vt + c * C::kDP * VS;
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
          ph[k] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);  // hi terms
          pl[k] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);  // lo terms
        }
        const v8bf bh8 = __builtin_bit_cast(v8bf, ph);
        const v8bf bl8 = __builtin_bit_cast(v8bf, pl);
#pragma unroll
        for (int t = 0; t < W; ++t) {
          v8bf av;
          if constexpr (VDIRECT) {
            av = v_operand(vt + c * 32 * 2 * C::kDP, t, ab);
          } else {
            const u32x4 vv = *reinterpret_cast<const u32x4*>(vt + c * C::kDP * VS + (32 * t + ql) * VS + 32 * half + 16 * ab);
            av = __builtin_bit_cast(v8bf, vv);
          }
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bh8, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bl8, acc[t], 0, 0, 0);
        }
      }
    }
  };

  // Tile of chunk gc (au = lutc + 2u per element) with every element that
  // this lane's row cannot see pushed up by kHidden: such an element then
  // fails the keep test and never equals auT, so the selection below needs
  // no visibility test of its own.  The adjustment runs only for the chunks
  // that some lane of the wave does not fully see.
  constexpr uint32_t kHidden = 2048;  // > 4*d_max + 4; au stays below 2^13
  auto attend_tile = [&](int buf, int c, int gc) {
    v16i t = logits_tile(buf, c, lutc);
    // chunks from wchunks on hold no key this wave sees (and from nchunk on,
    // half 0's slots would repeat half 1's keys)
    const int L = gc < wchunks ? lim - (half * Hh + 16 * gc) : 0;
    if (!__all(L >= 16)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) t[i] += (i < L) ? 0 : static_cast<int>(kHidden);
    }
    return t;
  };

  // Weight of element i of a chunk from its tile t.  Element i is kept iff
  // D = (au << 15) + sp < 0; the sign becomes a mask that selects au or the
  // zero slot, and the tie counter advances on au == auT: 5 vector ops.
  auto select_elem = [&](const v16i& t, int i, uint32_t* e) {
    const uint32_t au = static_cast<uint32_t>(t[i]);
    const uint32_t m = opaque(static_cast<uint32_t>(static_cast<int32_t>((au << 15) + sp) >> 31));
    e[i] = lds_load_u32((au & m) | (zaddr & ~m));
    sp = opaque(sp + ((au == auT) ? 1u : 0u));  // one compare + add-with-carry
  };
  auto select_chunk = [&](const v16i& t, uint32_t* e) {
#pragma unroll
    for (int i = 0; i < 16; ++i) select_elem(t, i, e);
  };

  // One key group, software-pipelined: every one of the kCH2 chunks is
  // processed (chunks past this wave's keys are entirely hidden and add
  // zero), and the selection of chunk c + 1 is interleaved in program order
  // with the 4W matrix-core products of chunk c (bf16 V): a product, then
  // 16/(4W) elements of vector work, so each product runs while the vector
  // ALU works and no product waits on its accumulator.  Unrolled over the
  // group so that consecutive chunks' weights live in distinct registers.
  auto attend_group = [&](int buf, int gi) {
    const unsigned char* vt = region + buf * C::kVBuf;
    const int g0 = gi * C::kCH2;
    if (wchunks - g0 <= 0) return;
    uint32_t e[C::kCH2][16];
    select_chunk(attend_tile(buf, 0, g0), e[0]);
    v16i tn = attend_tile(buf, C::kCH2 > 1 ? 1 : 0, g0 + (C::kCH2 > 1 ? 1 : 0));
#pragma unroll
    for (int c = 0; c < C::kCH2; ++c) {
      if constexpr (VF32) {
        if (c + 1 < C::kCH2) select_chunk(tn, e[c + 1]);
        pv_chunk(vt, c, e[c]);
      } else {
        // operands of chunk c's products: weights as bf16 hi / lo pairs, and
        // the transposed V tile pieces
        v8bf bh[2], bl[2], av[2][W];
#pragma unroll
        for (int ab = 0; ab < 2; ++ab) {
          u32x4 ph, pl;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t e0 = e[c][8 * ab + 2 * k], e1 = e[c][8 * ab + 2 * k + 1];
            ph[k] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);  // hi terms
            pl[k] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);  // lo terms
          }
          bh[ab] = __builtin_bit_cast(v8bf, ph);
          bl[ab] = __builtin_bit_cast(v8bf, pl);
#pragma unroll
          for (int t = 0; t < W; ++t) {
            if constexpr (VDIRECT) {
              av[ab][t] = v_operand(vt + c * 32 * 2 * C::kDP, t, ab);
            } else {
              const u32x4 vv = *reinterpret_cast<const u32x4*>(
                  vt + c * C::kDP * VS + (32 * t + ql) * VS + 32 * half + 16 * ab);
              av[ab][t] = __builtin_bit_cast(v8bf, vv);
            }
          }
        }
        constexpr int kProducts = 4 * W;
#pragma unroll
        for (int p = 0; p < kProducts; ++p) {
          const int ab = p / (2 * W), hl = (p / W) & 1, t = p % W;
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ab][t], hl ? bl[ab] : bh[ab], acc[t], 0, 0, 0);
          if (c + 1 < C::kCH2) {
#pragma unroll
            for (int i = (p * 16) / kProducts; i < ((p + 1) * 16) / kProducts; ++i) select_elem(tn, i, e[c + 1]);
          }
        }
      }
      if (c + 2 < C::kCH2) tn = attend_tile(buf, c + 2, g0 + c + 2);
    }
  };

  const int ngroups2 = (nchunk + C::kCH2 - 1) / C::kCH2;
  make_q(0x02u, 0xFCu);  // +-2: the tile holds au = lutc + 2u
  v_load(0);
  __syncthreads();  // every wave is done with its histogram (V tiles alias it)
  v_issue(0, 0);
  v_store(0);
  copies_done();
  for (int gi = 0; gi < ngroups2; ++gi) {
    const int buf = gi & 1;
    if (a.balance && (gi == 0 || gi == ngroups2 / 2 || gi == ngroups2 - 1))
      set_priority(gi == ngroups2 - 1 ? 0 : (gi < ngroups2 / 2 ? 2 : 1));
    if (gi + 1 < ngroups2) {
      k_issue((gi + 1) * C::kCH2, std::integral_constant<int, C::kCH2>{}, buf ^ 1);
      v_issue((gi + 1) * C::kCH2, buf ^ 1);
      v_load((gi + 1) * C::kCH2);
    }
    attend_group(buf, gi);
    if (gi + 1 < ngroups2) v_store(buf ^ 1);
    copies_done();
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

// Work-groups of this kernel the device holds at once (occupancy x CUs), per
// device and cached; 0 if the runtime cannot say.
template <int W, bool VF32, int MODE, bool VDIRECT>
int64_t resident_capacity() {
  static std::atomic<int64_t> cache[64];  // 0: not known yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int64_t cap = cache[dev].load(std::memory_order_relaxed);
  if (cap == 0) {
    using C = Cfg<W, VF32, VDIRECT>;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, had_attn_kernel<W, VF32, MODE, VDIRECT>,
                                                     C::kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    cap = static_cast<int64_t>(per_cu) * cus;
    cache[dev].store(cap, std::memory_order_relaxed);
  }
  return cap;
}

template <int W, bool VF32, int MODE, bool VDIRECT = false>
had_status launch_one(const AttnArgs& args, hipStream_t st) {
  using C = Cfg<W, VF32, VDIRECT>;
  const int qrows = (MODE == 2) ? args.row_count : args.n;
  const int64_t ntq = (qrows + C::kQB - 1) / C::kQB;
  const int64_t blocks = ntq * args.bh_count;
  if (blocks <= 0) return HAD_OK;
  if (blocks > 0x7FFFFFFF) return fail(HAD_ERR_UNSUPPORTED, "grid too large");
  AttnArgs a = args;
  a.balance = blocks <= resident_capacity<W, VF32, MODE, VDIRECT>() ? 1 : 0;
  had_attn_kernel<W, VF32, MODE, VDIRECT><<<static_cast<unsigned>(blocks), C::kThreads, 0, st>>>(a);
  return check_launch(MODE == 0   ? "had_attention"
                      : MODE == 1 ? "had_select"
                      : MODE == 2 ? "had_logits"
                      : MODE == 3 ? "had_topn_mass"
                                  : "had_backward (row statistics)");
}

template <int W>
had_status launch_w(AttnMode mode, const AttnArgs& a, hipStream_t st) {
  switch (mode) {
    case AttnMode::Attend:
      if (a.v_dtype == HAD_F32) return launch_one<W, true, 0>(a, st);
      // bf16 V with d a multiple of 32: rows copied straight into LDS
      if (a.d == 32 * W) return launch_one<W, false, 0, true>(a, st);
      return launch_one<W, false, 0>(a, st);
    case AttnMode::Select:
      return launch_one<W, false, 1>(a, st);
    case AttnMode::Logits:
      return launch_one<W, false, 2>(a, st);
    case AttnMode::Mass:
      return launch_one<W, false, 3>(a, st);
    case AttnMode::Stats:
      return launch_one<W, false, 4>(a, st);
  }
  return fail(HAD_ERR_INVALID_ARG, "unknown mode");
}

}  // namespace

int64_t attend_wave_count(const had_shape& s) {
  const int W = static_cast<int>(words_per_row(s.dim));
  const int waves = waves_for(W);
  return (s.seq + 32 * waves - 1) / (32 * waves) * s.batch * s.heads * waves;
}

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
