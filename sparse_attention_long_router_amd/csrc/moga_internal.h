// Internal helpers shared by the gfx950 kernels of libmoga.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moga.h"

namespace moga {

// ---- vector types -----------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxGroups = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, blocks dealt round-robin

// ---- bf16 <-> f32 -------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float32 -> two bf16 packed in a dword (lo = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// ---- launch-shape helpers -----------------------------------------------------
// Map a launch index to a work item so that each XCD receives runs of `run`
// consecutive items while the global order of runs is kept (blocks are dealt
// to XCDs round-robin).  Bijective on [0, grid) when grid % (kNumXcd*run) == 0.
__device__ __forceinline__ int xcd_remap(int b, int run) {
  const int x = b % kNumXcd, j = b / kNumXcd;
  return ((j / run) * kNumXcd + x) * run + (j % run);
}

}  // namespace moga

// ---- host-side helpers ------------------------------------------------------------
#define MOGA_LAUNCH_CHECK()                              \
  do {                                                   \
    if (hipGetLastError() != hipSuccess) return MOGA_ERR_HIP; \
  } while (0)

namespace moga {
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// Counting-sort geometry shared by the permute launcher and workspace sizing.
constexpr int kSortChunk = 1024;  // tokens per sort block
inline int64_t sort_blocks(int64_t N) { return ceil_div(N, kSortChunk); }

// Group-attention schedule record kept in workspace: groups in decreasing size
// and the prefix count of work items.
struct AttnSchedule {
  int32_t order[kMaxGroups];
  int32_t prefix[kMaxGroups + 1];
};

// Transposed-V layout Vt [H][D][ldv]: every channel row holds the N permuted
// tokens and zero padding up to ldv = N rounded up to 64, plus 64, so a
// 64-key tile starting at any key < N lies inside its row.  The attention
// kernel addresses one head's V^T rows with 32-bit offsets, (D-1)*ldv*2 + 128
// bytes, which bounds N.
inline int64_t vt_row_length(int64_t N) { return (N + 63) / 64 * 64 + 64; }
constexpr int64_t kVtMaxTokens = (int64_t(1) << 23) - 128;

inline bool valid_head_dims(int32_t H, int32_t D) {
  return H >= 1 && (D == 64 || D == 128) && (int64_t)H * D <= 8192;
}
}  // namespace moga

// Router-logit gradient from the route kernel (route.hip), used by
// moga_route_backward: dlogits [N, M] float.
int moga_route_dlogits(const uint16_t* x, const uint16_t* w, const float* bias, int64_t N, int32_t d_model, int32_t M,
                       const int32_t* group_id, const float* dgate, float* dlogits, hipStream_t st);
