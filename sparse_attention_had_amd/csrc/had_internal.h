// Internal declarations shared by the HIP translation units of libhad.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
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

// Shape checks common to every entry point.
had_status check_shape(const had_shape& s);

// ---- pack ----
int pack_grid_blocks(const had_shape& s);

// ---- attention family (had_attention.hip) ----
enum class AttnMode : int { Attend = 0, Select = 1, Logits = 2 };

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
};

had_status launch_attention_family(AttnMode mode, const AttnArgs& a, hipStream_t st);

}  // namespace had
