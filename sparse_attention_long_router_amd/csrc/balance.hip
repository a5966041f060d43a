// Group-balancing statistics of the router: F_i, P_i and
// L_gb = alpha * M * sum_i F_i P_i.
// Page "MoGA: Mixture-of-Groups Attention for End-to-End Long Video
// Generation", section "Group Balancing Loss: Preventing Router Collapse"
// (Eq. 6): F_i is the fraction of tokens assigned to group i, and P_i the
// routing probability of the assigned tokens summed over group i and divided
// by N, as the equation writes it.
//
// Deterministic two-pass reduction (no float atomics): each 1024-token block
// reduces per-group counts (ballot + popcount) and gate sums (wave butterfly)
// in a fixed order, then one workgroup adds the block partials in block order.
#include "moga_internal.h"

namespace moga {
namespace {

constexpr int kBalThreads = 256;
constexpr int kBalWaves = kBalThreads / kWave;

__global__ __launch_bounds__(kBalThreads) void balance_partial_kernel(const int32_t* __restrict__ gid,
                                                                    const float* __restrict__ gate, int64_t N, int M,
                                                                    int nblk, int32_t* __restrict__ cnt,
                                                                    float* __restrict__ psum) {
  __shared__ int wc[kBalWaves][kMaxGroups];
  __shared__ float ws[kBalWaves][kMaxGroups];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int my_c = 0;  // lane g of the wave keeps group g (M <= 64)
  float my_s = 0.f;
  const int64_t n0 = (int64_t)blockIdx.x * kSortChunk;
  for (int r0 = wave * kWave; r0 < kSortChunk; r0 += kBalThreads) {
    const int64_t n = n0 + r0 + lane;
    const bool valid = n < N;
    const int g = valid ? gid[n] : -1;
    const float p = valid ? gate[n] : 0.f;
    for (int i = 0; i < M; ++i) {
      const bool mine = g == i;
      const int c = __popcll(__ballot(mine));
      float v = mine ? p : 0.f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      if (lane == i) {
        my_c += c;
        my_s += v;
      }
    }
  }
  if (lane < M) {
    wc[wave][lane] = my_c;
    ws[wave][lane] = my_s;
  }
  __syncthreads();
  if (threadIdx.x < M) {
    int c = 0;
    float v = 0.f;
    for (int w = 0; w < kBalWaves; ++w) {
      c += wc[w][threadIdx.x];
      v += ws[w][threadIdx.x];
    }
    cnt[(int64_t)threadIdx.x * nblk + blockIdx.x] = c;
    psum[(int64_t)threadIdx.x * nblk + blockIdx.x] = v;
  }
}

__global__ __launch_bounds__(kWave) void balance_final_kernel(const int32_t* __restrict__ cnt,
                                                             const float* __restrict__ psum, int64_t N, int M,
                                                             int nblk, float alpha, float* __restrict__ F,
                                                             float* __restrict__ P, float* __restrict__ loss) {
  const int g = threadIdx.x;
  float fp = 0.f;
  if (g < M) {
    int64_t c = 0;
    float v = 0.f;
    for (int b = 0; b < nblk; ++b) {
      c += cnt[(int64_t)g * nblk + b];
      v += psum[(int64_t)g * nblk + b];
    }
    const float f = (float)((double)c / (double)N);
    const float pg = v / (float)N;
    F[g] = f;
    P[g] = pg;
    fp = f * pg;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) fp += __shfl_xor(fp, off);
  if (g == 0) *loss = alpha * (float)M * fp;
}

}  // namespace
}  // namespace moga

extern "C" int moga_balance_stats(const int32_t* group_id, const float* gate, int64_t N, int32_t M, float alpha,
                                  float* F, float* P, float* loss, void* ws, size_t ws_bytes, void* stream) {
  using namespace moga;
  if (!group_id || !gate || !F || !P || !loss) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups) return MOGA_ERR_UNSUPPORTED;
  const size_t need = moga_workspace_bytes(MOGA_OP_BALANCE_STATS, N, M, 1, 64);
  if (!ws || ws_bytes < need) return MOGA_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  const int nblk = (int)sort_blocks(N);
  int32_t* cnt = static_cast<int32_t*>(ws);
  float* psum = reinterpret_cast<float*>(cnt + (size_t)M * nblk);
  balance_partial_kernel<<<nblk, kBalThreads, 0, st>>>(group_id, gate, N, M, nblk, cnt, psum);
  MOGA_LAUNCH_CHECK();
  balance_final_kernel<<<1, kWave, 0, st>>>(cnt, psum, N, M, nblk, alpha, F, P, loss);
  MOGA_LAUNCH_CHECK();
  return MOGA_OK;
}
