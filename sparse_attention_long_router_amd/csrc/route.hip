// Router kernel: scores r = X W_r^T (+bias) with bf16 MFMA, then the hard
// assignment g = argmax r and the gate p(g|x) = 1 / sum_j exp(r_j - r_g).
// Page "MoGA: Mixture-of-Groups Attention for End-to-End Long Video
// Generation", section "MoGA Router" (routing scores, Eq. 3, argmax) and the
// MoGA output equation in "Grouped Attention".
//
// Shape of the work: M <= 64 groups against d_model up to thousands, so each
// token costs 2*M flops per 2 bytes of X read -- far below the MFMA ridge.  The
// kernel is an HBM stream over X; MFMA is used so the arithmetic stays well
// under the streaming time (plain fp32 VALU FMAs would not at M = 16..64).
//
// MFMA v_mfma_f32_16x16x32_bf16 computes C^T = W_r X^T per 16 tokens:
//   A = W_r fragment (16 groups x 32 k), B = X^T fragment (32 k x 16 tokens),
//   lane (q = lane/16, c = lane%16) feeds A row c / B column c with the 8
//   k-values of slot q; C reg r holds group 4q+r of token c.
// Per 128-channel step each lane issues four 16-byte loads: load j covers
// channels j*32 + q*8 .. +7 of its token, so one load instruction reads 64
// contiguous bytes of each of 16 token rows (the four lane quads take adjacent
// chunks) and the four loads together cover 256 contiguous bytes per row.
#include "moga_internal.h"

namespace moga {
namespace {

constexpr int kRouteWaves = 4;
constexpr int kRouteTokBlocks = 4;  // 16-token blocks per wave
constexpr int kRouteTokensPerBlock = kRouteWaves * kRouteTokBlocks * 16;  // 256

// kGrad = false: group_id and gate out.  kGrad = true (backward): group_id
// and dgate in, and the router-logit gradient out,
//   dlogits[t][j] = dgate[t] * p_g * ([j == g] - p_j),  p = softmax(r_t),
// the derivative of the gate p_g (Eq. 3) with the hard choice g held fixed.
template <int MB, bool kGrad>  // ceil(M / 16) group blocks
__global__ __launch_bounds__(kRouteWaves * kWave) void route_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
    int64_t N, int dm, int M, int32_t* __restrict__ group_id, float* __restrict__ gate,
    const float* __restrict__ dgate, float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, c = lane & 15;
  const int64_t tok0 = (int64_t)blockIdx.x * kRouteTokensPerBlock + wave * (kRouteTokBlocks * 16);

  const uint16_t* xrow[kRouteTokBlocks];
#pragma unroll
  for (int tb = 0; tb < kRouteTokBlocks; ++tb) {
    int64_t t = tok0 + tb * 16 + c;
    t = t < N ? t : N - 1;  // clamp: rows past N are computed but never stored
    xrow[tb] = X + t * dm;
  }
  const uint16_t* wrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    int g = mb * 16 + c;
    g = g < M ? g : M - 1;  // padded groups are masked in the epilogue
    wrow[mb] = Wr + (int64_t)g * dm;
  }

  f32x4 acc[kRouteTokBlocks][MB];
#pragma unroll
  for (int tb = 0; tb < kRouteTokBlocks; ++tb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[tb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // main loop: 128 channels per step, software-pipelined so the loads of step
  // k+1 are in flight while step k's MFMAs run
  const int nmain = dm / 128;
  bf16x8 xf[2][kRouteTokBlocks][4], wf[2][MB][4];
  auto load_step = [&](int buf, int kbase) {
    const int kq = kbase + q * 8;
#pragma unroll
    for (int tb = 0; tb < kRouteTokBlocks; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xf[buf][tb][j] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(xrow[tb] + kq + j * 32));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) wf[buf][mb][j] = *reinterpret_cast<const bf16x8*>(wrow[mb] + kq + j * 32);
  };
  auto mfma_step = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int tb = 0; tb < kRouteTokBlocks; ++tb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[tb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[buf][mb][j], xf[buf][tb][j], acc[tb][mb], 0, 0, 0);
  };
  if (nmain > 0) load_step(0, 0);
  int i = 0;
  for (; i + 2 <= nmain; i += 2) {
    load_step(1, (i + 1) * 128);
    mfma_step(0);
    if (i + 2 < nmain) load_step(0, (i + 2) * 128);
    mfma_step(1);
  }
  if (i < nmain) mfma_step(0);
  int k0 = nmain * 128;
  // tail: 32 channels per step (d_model is a multiple of 32)
  for (; k0 < dm; k0 += 32) {
    const int kq = k0 + q * 8;
#pragma unroll
    for (int tb = 0; tb < kRouteTokBlocks; ++tb) {
      bf16x8 xv = *reinterpret_cast<const bf16x8*>(xrow[tb] + kq);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        bf16x8 wv = *reinterpret_cast<const bf16x8*>(wrow[mb] + kq);
        acc[tb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, xv, acc[tb][mb], 0, 0, 0);
      }
    }
  }

  // epilogue: per token, argmax (lowest index on ties) and gate
#pragma unroll
  for (int tb = 0; tb < kRouteTokBlocks; ++tb) {
    float r[MB][4];
    float best = -INFINITY;
    int besti = 0x7fffffff;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = mb * 16 + q * 4 + i;
        float v = acc[tb][mb][i];
        if (g < M) {
          if (bias) v += bias[g];
        } else {
          v = -INFINITY;
        }
        r[mb][i] = v;
        if (v > best) { best = v; besti = g; }  // groups visited in increasing id
      }
    // combine the four lane quads holding this token's other groups
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float ob = __shfl_xor(best, off);
      const int oi = __shfl_xor(besti, off);
      if (ob > best || (ob == best && oi < besti)) { best = ob; besti = oi; }
    }
    float s = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s += expf(r[mb][i] - best);  // masked: exp(-inf) = 0
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    const int64_t t = tok0 + tb * 16 + c;
    if constexpr (!kGrad) {
      if (q == 0 && t < N) {
        group_id[t] = besti;
        gate[t] = 1.0f / s;
      }
    } else {
      const int64_t tc = t < N ? t : N - 1;
      const int g = group_id[tc];
      const float inv = 1.0f / s;
      float pg = 0.f;  // p of the chosen group, gathered from the lane quad that holds it
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (mb * 16 + q * 4 + i == g) pg = expf(r[mb][i] - best) * inv;
      pg += __shfl_xor(pg, 16);
      pg += __shfl_xor(pg, 32);
      const float f = dgate[tc] * pg;
      if (t < N) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = mb * 16 + q * 4 + i;
            if (j < M) dlogits[t * M + j] = f * ((j == g ? 1.f : 0.f) - expf(r[mb][i] - best) * inv);
          }
      }
    }
  }
}

template <int MB, bool kGrad = false>
void launch_route(const uint16_t* X, const uint16_t* Wr, const float* bias, int64_t N, int dm, int M,
                  int32_t* gid, float* gate, hipStream_t st, const float* dgate = nullptr,
                  float* dlogits = nullptr) {
  const int64_t blocks = ceil_div(N, kRouteTokensPerBlock);
  route_kernel<MB, kGrad><<<dim3((unsigned)blocks), dim3(kRouteWaves * kWave), 0, st>>>(X, Wr, bias, N, dm, M, gid,
                                                                                       gate, dgate, dlogits);
}

}  // namespace
}  // namespace moga

extern "C" int moga_route(const void* X, const void* Wr, const float* bias, int64_t N, int32_t d_model,
                          int32_t M, int32_t* group_id, float* gate, void* stream) {
  using namespace moga;
  if (!X || !Wr || !group_id || !gate) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1 || d_model < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups || d_model % 32 != 0) return MOGA_ERR_UNSUPPORTED;
  const auto* x = static_cast<const uint16_t*>(X);
  const auto* w = static_cast<const uint16_t*>(Wr);
  hipStream_t st = as_stream(stream);
  switch ((M + 15) / 16) {
    case 1: launch_route<1>(x, w, bias, N, d_model, M, group_id, gate, st); break;
    case 2: launch_route<2>(x, w, bias, N, d_model, M, group_id, gate, st); break;
    case 3: launch_route<3>(x, w, bias, N, d_model, M, group_id, gate, st); break;
    default: launch_route<4>(x, w, bias, N, d_model, M, group_id, gate, st); break;
  }
  MOGA_LAUNCH_CHECK();
  return MOGA_OK;
}

// Router-logit gradient (backward of the gate); internal entry used by
// moga_route_backward.
int moga_route_dlogits(const uint16_t* x, const uint16_t* w, const float* bias, int64_t N, int32_t d_model, int32_t M,
                       const int32_t* group_id, const float* dgate, float* dlogits, hipStream_t st) {
  using namespace moga;
  int32_t* gid = const_cast<int32_t*>(group_id);  // read only when kGrad
  switch ((M + 15) / 16) {
    case 1: launch_route<1, true>(x, w, bias, N, d_model, M, gid, nullptr, st, dgate, dlogits); break;
    case 2: launch_route<2, true>(x, w, bias, N, d_model, M, gid, nullptr, st, dgate, dlogits); break;
    case 3: launch_route<3, true>(x, w, bias, N, d_model, M, gid, nullptr, st, dgate, dlogits); break;
    default: launch_route<4, true>(x, w, bias, N, d_model, M, gid, nullptr, st, dgate, dlogits); break;
  }
  MOGA_LAUNCH_CHECK();
  return MOGA_OK;
}
