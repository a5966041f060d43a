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
//
// Streaming: HBM delivers far more when every load instruction reads long
// contiguous runs of a row.  Loading X straight in the MFMA layout (16 token
// rows x 64 bytes per instruction) measured about 5.2 TB/s; 4 rows x 256
// contiguous bytes per instruction measured about 6.8 TB/s.  So each wave
// loads its rows in the wide form -- lane l takes 16-byte chunk l%16 of row
// l/16 of a 4-row group -- into a register ring several 128-channel steps
// deep, and re-lays each step out through its own LDS buffer: chunk p of row
// r is stored at chunk p ^ (r % 16), which keeps both the row-wise writes and
// the MFMA-layout reads (16 rows, one chunk each) free of bank conflicts.
// The LDS buffer is private to the wave, so no barrier is needed: one wave's
// LDS operations complete in order.
#include "moga_internal.h"

typedef int32_t i32x4v __attribute__((ext_vector_type(4)));
// LLVM's raw buffer loads of 16 bytes: descriptor, per-lane byte offset,
// scalar byte offset, cache policy.  Offsets past the descriptor's range read
// zeros.  The bf16 form feeds MFMA operands straight from the load (a bit cast
// from the integer form costs no-op VALU moves that wait on the load).
__device__ moga::u32x4 raw_buffer_load_x4(i32x4v rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ moga::bf16x8 raw_buffer_load_bf16x8(i32x4v rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v8bf16");

namespace moga {
namespace {

constexpr int kRouteWaves = 4;
constexpr int kCpolNt = 2;  // non-temporal: X is read once

__device__ __forceinline__ i32x4v range_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int64_t range = bytes < 0 ? 0 : (bytes < 0xffffffffll ? bytes : 0xffffffffll);
  i32x4v r;
  r[0] = (int32_t)(uint32_t)a;
  r[1] = (int32_t)(uint32_t)(a >> 32);
  r[2] = (int32_t)(uint32_t)range;
  r[3] = 0x00020000;
  return r;
}

// kGrad = false: group_id and gate out.  kGrad = true (backward): group_id
// and dgate in, and the router-logit gradient out,
//   dlogits[t][j] = dgate[t] * p_g * ([j == g] - p_j),  p = softmax(r_t),
// the derivative of the gate p_g (Eq. 3) with the hard choice g held fixed.
// TB: 16-token blocks per wave; DEPTH: 128-channel steps in flight per wave.
template <int MB, int TB, int DEPTH, bool kGrad>  // MB = ceil(M / 16) group blocks
__global__ __launch_bounds__(kRouteWaves * kWave) void route_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wr, const float* __restrict__ bias,
    int64_t N, int dm, int M, int32_t* __restrict__ group_id, float* __restrict__ gate,
    const float* __restrict__ dgate, float* __restrict__ dlogits) {
  constexpr int TW = TB * 16;   // tokens per wave
  constexpr int NI = TW / 4;    // wide load instructions per 128-channel step
  __shared__ __attribute__((aligned(16))) uint16_t lds_all[kRouteWaves][TW * 128];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4, c = lane & 15;
  const int64_t tok0 = ((int64_t)blockIdx.x * kRouteWaves + wave) * TW;
  const int rowb = dm * 2;
  int64_t nrows = N - tok0;
  nrows = nrows < 0 ? 0 : (nrows < TW ? nrows : TW);
  const i32x4v xrs = range_rsrc(X + tok0 * dm, nrows * rowb);    // this wave's rows; the rest read as zeros
  const i32x4v wrs = range_rsrc(Wr, (int64_t)M * rowb);          // padded groups read as zeros
  uint16_t* lds = lds_all[wave];

  f32x4 acc[TB][MB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[tb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // wide load: instruction i covers rows 4i..4i+3; lane (q, c) reads row 4i+q, chunk c
  const int xv0 = q * rowb + c * 16;
  // W: lane (q, c) of group block mb reads group mb*16+c, chunk 4j+q of the step (j = immediate 64*j)
  const int wv0 = c * rowb + q * 16;
  // LDS write address of instruction i (row 4i+q, chunk c ^ row%16): depends on i%4; i/4 adds 16 rows
  int wa[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) wa[k] = (4 * k + q) * 256 + ((c ^ (4 * k + q)) * 16);
  // LDS read address of MFMA slot j (row 16tb+c, chunk (4j+q) ^ c); tb adds 16 rows
  int ra[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ra[j] = c * 256 + (((4 * j + q) ^ c) * 16);

  u32x4 xr[DEPTH][NI];
  bf16x8 wf[DEPTH][MB][4];
  const int nmain = dm / 128;
  auto load_step = [&](u32x4(&xs)[NI], bf16x8(&ws)[MB][4], int s) {
    const int so = s * 256;
#pragma unroll
    for (int i = 0; i < NI; ++i) xs[i] = raw_buffer_load_x4(xrs, xv0 + i * 4 * rowb + so, 0, kCpolNt);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ws[mb][j] = raw_buffer_load_bf16x8(wrs, wv0 + mb * 16 * rowb + j * 64 + so, 0, 0);
  };
  auto compute_step = [&](u32x4(&xs)[NI], bf16x8(&ws)[MB][4]) {
    char* lb = reinterpret_cast<char*>(lds);
#pragma unroll
    for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(lb + wa[i & 3] + (i >> 2) * 4096) = xs[i];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      bf16x8 xf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[j] = *reinterpret_cast<const bf16x8*>(lb + ra[j] + tb * 4096);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[tb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ws[mb][j], xf[j], acc[tb][mb], 0, 0, 0);
    }
  };
  // The steady loop issues every load unconditionally, so each step waits
  // only for its own slot while the other DEPTH-1 slots stay in flight.
  int s0 = 0;
  if (nmain >= DEPTH) {
#pragma unroll
    for (int b = 0; b < DEPTH; ++b) load_step(xr[b], wf[b], b);
    for (; s0 + 2 * DEPTH <= nmain; s0 += DEPTH) {
#pragma unroll
      for (int b = 0; b < DEPTH; ++b) {
        compute_step(xr[b], wf[b]);
        load_step(xr[b], wf[b], s0 + DEPTH + b);
      }
    }
    // drain: slots hold steps s0 .. s0+DEPTH-1; fewer than DEPTH steps follow
#pragma unroll
    for (int b = 0; b < DEPTH; ++b) {
      compute_step(xr[b], wf[b]);
      if (s0 + DEPTH + b < nmain) load_step(xr[b], wf[b], s0 + DEPTH + b);
    }
#pragma unroll
    for (int b = 0; b < DEPTH; ++b)
      if (s0 + DEPTH + b < nmain) compute_step(xr[b], wf[b]);
  } else {
    for (; s0 < nmain; ++s0) {
      load_step(xr[0], wf[0], s0);
      compute_step(xr[0], wf[0]);
    }
  }
  // tail: 32 channels per step (d_model is a multiple of 32), loaded straight in the MFMA layout
  for (int k0 = nmain * 128; k0 < dm; k0 += 32) {
    bf16x8 wv[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      wv[mb] = raw_buffer_load_bf16x8(wrs, wv0 + mb * 16 * rowb + k0 * 2, 0, 0);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const bf16x8 xv = raw_buffer_load_bf16x8(xrs, (tb * 16 + c) * rowb + k0 * 2 + q * 16, 0, kCpolNt);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[tb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[mb], xv, acc[tb][mb], 0, 0, 0);
    }
  }

  // epilogue: per token, argmax (lowest index on ties) and gate
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
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
  // 16-token blocks per wave: as many as keep two waves per SIMD once the
  // accumulators and W fragments grow with M (measured at d_model 1536/5120:
  // 64 tokens per wave beat 32 at M = 16; at M = 32, 32 beat 16 and 64)
  constexpr int TB = MB == 1 ? 4 : (MB == 2 ? 2 : 1);
  constexpr int DEPTH = 2;  // steps in flight; 3 and 4 measured no faster
  const int64_t blocks = ceil_div(N, (int64_t)kRouteWaves * TB * 16);
  route_kernel<MB, TB, DEPTH, kGrad><<<dim3((unsigned)blocks), dim3(kRouteWaves * kWave), 0, st>>>(
      X, Wr, bias, N, dm, M, gid, gate, dgate, dlogits);
}

}  // namespace
}  // namespace moga

extern "C" int moga_route(const void* X, const void* Wr, const float* bias, int64_t N, int32_t d_model,
                          int32_t M, int32_t* group_id, float* gate, void* ws, size_t ws_bytes, void* stream) {
  using namespace moga;
  (void)ws;  // the route needs no workspace (moga_workspace_bytes(MOGA_OP_ROUTE, ...) == 0)
  (void)ws_bytes;
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
