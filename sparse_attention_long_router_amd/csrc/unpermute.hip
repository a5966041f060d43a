// Gate-scaled unpermute: O[perm[j]] = beta * O[perm[j]] + gate[perm[j]] * Op[j].
// Page "MoGA: Mixture-of-Groups Attention for End-to-End Long Video
// Generation": the MoGA output equation ("Grouped Attention" section)
// multiplies a token's in-group attention by its routing probability, and
// Algorithm 1 step 4 returns rows to the original token order.
//
// HBM-bound stream of whole H*D rows: one wave per row, 16-byte lanes, float32
// arithmetic and one round-to-nearest-even bf16 store.
#include "moga_internal.h"

namespace moga {
namespace {

constexpr int kUnpermWaves = 4;
constexpr int kUnpermRows = 16;

template <bool kAccumulate>
__global__ __launch_bounds__(kUnpermWaves * kWave) void unpermute_kernel(
    const u32x4* __restrict__ Op, const int32_t* __restrict__ perm, const float* __restrict__ gate, int64_t N,
    int chunks, float beta, u32x4* __restrict__ O) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j0 = (int64_t)blockIdx.x * kUnpermRows;
  for (int rr = wave; rr < kUnpermRows; rr += kUnpermWaves) {
    const int64_t j = j0 + rr;
    if (j >= N) break;
    const int32_t n = perm[j];
    const float gv = gate[n];
    const int64_t src = j * chunks, dst = (int64_t)n * chunks;
    for (int c = lane; c < chunks; c += kWave) {
      const u32x4 a = __builtin_nontemporal_load(Op + src + c);
      u32x4 out;
      if constexpr (kAccumulate) {
        const u32x4 b = O[dst + c];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          out[i] = pack_bf16x2(beta * bf16_lo(b[i]) + gv * bf16_lo(a[i]), beta * bf16_hi(b[i]) + gv * bf16_hi(a[i]));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = pack_bf16x2(gv * bf16_lo(a[i]), gv * bf16_hi(a[i]));
      }
      __builtin_nontemporal_store(out, O + dst + c);
    }
  }
}

}  // namespace
}  // namespace moga

extern "C" int moga_unpermute(const void* Op, const int32_t* perm, const float* gate, int64_t N, int32_t H,
                              int32_t D, float beta, void* O, void* stream) {
  using namespace moga;
  if (!Op || !perm || !gate || !O) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || H < 1 || D < 1) return MOGA_ERR_SHAPE;
  if (!valid_head_dims(H, D)) return MOGA_ERR_UNSUPPORTED;
  const int chunks = H * D / 8;
  const int64_t blocks = ceil_div(N, kUnpermRows);
  hipStream_t st = as_stream(stream);
  const auto* op = static_cast<const u32x4*>(Op);
  auto* o = static_cast<u32x4*>(O);
  if (beta == 0.0f)
    unpermute_kernel<false><<<dim3((unsigned)blocks), kUnpermWaves * kWave, 0, st>>>(op, perm, gate, N, chunks, beta, o);
  else
    unpermute_kernel<true><<<dim3((unsigned)blocks), kUnpermWaves * kWave, 0, st>>>(op, perm, gate, N, chunks, beta, o);
  MOGA_LAUNCH_CHECK();
  return MOGA_OK;
}
