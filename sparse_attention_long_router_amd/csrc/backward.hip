// Backward of the gated unpermute and of the router.
// Page "MoGA: Mixture-of-Groups Attention for End-to-End Long Video
// Generation", "Grouped Attention" section: the output is
// p(g(x)|x) * SA(x) and the gate p is the router's gradient path (the hard
// argmax has none); "MoGA Router" section: p = softmax(x W_r^T + b) (Eq. 3).
// For L = sum(O * dO):
//   dgate[n]      = <dO[n], SA[n]>                 (over heads and channels)
//   dA[j]         = gate[n] * dO[n],  n = perm[j]  (permuted, for the attention)
//   delta[h][j]   = <dA[j, h], SA[j, h]>           (row sums the attention backward needs,
//                   from the bf16-rounded dA the attention backward reads, so that
//                   dP - delta cancels where it should, e.g. in one-token groups)
//   dlogits[n][j] = dgate[n] * p_g * ([j == g] - p_j)
//   dX = dlogits W_r,  dW_r = dlogits^T X,  db = sum_n dlogits[n].
// All reductions run in a fixed order (no float atomics), so results are
// bitwise repeatable.
#include "moga_internal.h"

namespace moga {
namespace {

constexpr int kUbWaves = 4;

// One wave per permuted row: 8 channels per lane and pass; a head covers D/8
// consecutive lanes, reduced with butterflies inside that lane group.
__global__ __launch_bounds__(kUbWaves * kWave) void unpermute_backward_kernel(
    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ Op, const int32_t* __restrict__ perm,
    const float* __restrict__ gate, int64_t N, int H, int D, uint16_t* __restrict__ dA, float* __restrict__ delta,
    float* __restrict__ dgate) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * kUbWaves + (threadIdx.x >> 6);
  if (j >= N) return;  // uniform per wave
  const int64_t n = perm[j];
  const float gn = gate[n];
  const int row = H * D;
  const int G = D / 8;  // lanes per head within a pass
  float total = 0.f;
  for (int e0 = lane * 8; e0 - lane * 8 < row; e0 += kWave * 8) {
    float part = 0.f, dpart = 0.f;
    if (e0 < row) {
      const u32x4 o = *reinterpret_cast<const u32x4*>(dO + n * row + e0);
      const u32x4 a = *reinterpret_cast<const u32x4*>(Op + j * row + e0);
      u32x4 out;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float o0 = bf16_lo(o[k]), o1 = bf16_hi(o[k]);
        const float a0 = bf16_lo(a[k]), a1 = bf16_hi(a[k]);
        part += o0 * a0 + o1 * a1;
        out[k] = pack_bf16x2(gn * o0, gn * o1);
        dpart += bf16_lo(out[k]) * a0 + bf16_hi(out[k]) * a1;
      }
      *reinterpret_cast<u32x4*>(dA + j * row + e0) = out;
    }
    float hsum = dpart;
    for (int off = G >> 1; off >= 1; off >>= 1) hsum += __shfl_xor(hsum, off);
    if (e0 < row && (lane % G) == 0) delta[(int64_t)(e0 / D) * N + j] = hsum;
    total += part;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) total += __shfl_xor(total, off);
  if (lane == 0) dgate[n] = total;
}

constexpr int kChan = 256;      // channels per block (one per thread)
constexpr int kDxTokens = 64;   // tokens per dX block
constexpr int kDwTokens = 1024; // tokens per dW_r partial block
constexpr int kDwStage = 128;   // dlogits rows staged in LDS at a time
constexpr int kDwUnroll = 16;   // X rows loaded ahead of their FMAs

// dX[n][c] = sum_j dlogits[n][j] * W_r[j][c]: a thread owns channel c and
// keeps W_r[:, c] in registers; the block's dlogits rows sit in LDS.
template <int MB>
__global__ __launch_bounds__(kChan) void router_dx_kernel(const float* __restrict__ dl, const uint16_t* __restrict__ Wr,
                                                         int64_t N, int dm, int M, float* __restrict__ dX) {
  __shared__ float dls[kDxTokens * MB * 16];
  const int c = blockIdx.y * kChan + threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * kDxTokens;
  for (int i = threadIdx.x; i < kDxTokens * MB * 16; i += kChan) {
    const int t = i / (MB * 16), jj = i % (MB * 16);
    dls[i] = (n0 + t < N && jj < M) ? dl[(n0 + t) * M + jj] : 0.f;
  }
  float w[MB * 16];
#pragma unroll
  for (int jj = 0; jj < MB * 16; ++jj) {
    const uint16_t h = (c < dm && jj < M) ? Wr[(int64_t)jj * dm + c] : (uint16_t)0;
    w[jj] = __uint_as_float((uint32_t)h << 16);
  }
  __syncthreads();
  if (c >= dm) return;
  for (int t = 0; t < kDxTokens && n0 + t < N; ++t) {
    float acc = 0.f;
#pragma unroll
    for (int jj = 0; jj < MB * 16; jj += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(&dls[t * MB * 16 + jj]);
      acc = fmaf(v[0], w[jj], acc);
      acc = fmaf(v[1], w[jj + 1], acc);
      acc = fmaf(v[2], w[jj + 2], acc);
      acc = fmaf(v[3], w[jj + 3], acc);
    }
    dX[(n0 + t) * dm + c] = acc;
  }
}

// Partial dW_r (and db) of one block of kDwTokens tokens:
// part[blk][j][c] = sum_n dlogits[n][j] * X[n][c], dbp[blk][j] = sum_n dlogits[n][j].
// A thread owns CPT consecutive channels (one 2*CPT-byte load of X per token)
// and keeps 16*MB*CPT accumulators; the block's dlogits rows are staged in
// LDS and read as float4 broadcasts, and the X loads of kDwUnroll tokens are
// in flight before their FMAs.  Each channel sums its tokens in token order,
// so the partials do not depend on CPT or the unrolling.  At d_model 1536,
// M = 16 the router backward measured 1.07 ms with one channel per thread and
// one token at a time, 0.61 ms with two channels and 16 tokens ahead (four
// channels: 0.69 ms, fewer workgroups in flight).
template <int MB>
constexpr int dw_cpt() { return MB <= 2 ? 2 : 1; }

template <int MB>
__global__ __launch_bounds__(kChan) void router_dw_partial_kernel(const float* __restrict__ dl,
                                                                 const uint16_t* __restrict__ X, int64_t N, int dm,
                                                                 int M, float* __restrict__ part,
                                                                 float* __restrict__ dbp) {
  constexpr int CPT = dw_cpt<MB>();
  __shared__ float dls[kDwStage * MB * 16];
  const int c0 = (blockIdx.y * kChan + threadIdx.x) * CPT;  // dm is a multiple of 32: CPT channels all in or out
  const int64_t n0 = (int64_t)blockIdx.x * kDwTokens;
  float acc[MB * 16][CPT];
#pragma unroll
  for (int jj = 0; jj < MB * 16; ++jj)
#pragma unroll
    for (int k = 0; k < CPT; ++k) acc[jj][k] = 0.f;
  float bacc = 0.f;  // threads jj < M of the first channel slice: db
  for (int s0 = 0; s0 < kDwTokens; s0 += kDwStage) {
    __syncthreads();
    for (int i = threadIdx.x; i < kDwStage * MB * 16; i += kChan) {
      const int t = i / (MB * 16), jj = i % (MB * 16);
      const int64_t n = n0 + s0 + t;
      dls[i] = (n < N && jj < M) ? dl[n * M + jj] : 0.f;
    }
    __syncthreads();
    if (blockIdx.y == 0 && threadIdx.x < M)
      for (int t = 0; t < kDwStage; ++t) bacc += dls[t * MB * 16 + threadIdx.x];
    if (c0 < dm) {
      // kDwUnroll tokens' X loads in flight at once (rows past N read row N-1
      // and meet zero dlogits, so they add nothing)
      for (int t0 = 0; t0 < kDwStage; t0 += kDwUnroll) {
        float x[kDwUnroll][CPT];
#pragma unroll
        for (int u = 0; u < kDwUnroll; ++u) {
          int64_t n = n0 + s0 + t0 + u;
          n = n < N ? n : N - 1;
          const uint16_t* xp = X + n * dm + c0;
          if constexpr (CPT == 4) {
            const u32x2 v = *reinterpret_cast<const u32x2*>(xp);
            x[u][0] = bf16_lo(v[0]); x[u][1] = bf16_hi(v[0]); x[u][2] = bf16_lo(v[1]); x[u][3] = bf16_hi(v[1]);
          } else if constexpr (CPT == 2) {
            const uint32_t v = *reinterpret_cast<const uint32_t*>(xp);
            x[u][0] = bf16_lo(v); x[u][1] = bf16_hi(v);
          } else {
            x[u][0] = __uint_as_float((uint32_t)xp[0] << 16);
          }
        }
#pragma unroll
        for (int u = 0; u < kDwUnroll; ++u) {
          const int t = t0 + u;
#pragma unroll
          for (int jj = 0; jj < MB * 16; jj += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(&dls[t * MB * 16 + jj]);
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
              acc[jj][k] = fmaf(v[0], x[u][k], acc[jj][k]);
              acc[jj + 1][k] = fmaf(v[1], x[u][k], acc[jj + 1][k]);
              acc[jj + 2][k] = fmaf(v[2], x[u][k], acc[jj + 2][k]);
              acc[jj + 3][k] = fmaf(v[3], x[u][k], acc[jj + 3][k]);
            }
          }
        }
      }
    }
  }
  if (c0 < dm) {
#pragma unroll
    for (int jj = 0; jj < MB * 16; ++jj)
      if (jj < M) {
        float* out = part + ((int64_t)blockIdx.x * M + jj) * dm + c0;
#pragma unroll
        for (int k = 0; k < CPT; ++k) out[k] = acc[jj][k];
      }
  }
  if (blockIdx.y == 0 && threadIdx.x < M) dbp[(int64_t)blockIdx.x * M + threadIdx.x] = bacc;
}

// dW_r[j][c] = sum over blocks in block order; db likewise.
__global__ __launch_bounds__(kChan) void router_dw_reduce_kernel(const float* __restrict__ part,
                                                                const float* __restrict__ dbp, int nblk, int dm, int M,
                                                                float* __restrict__ dWr, float* __restrict__ db) {
  const int64_t i = (int64_t)blockIdx.x * kChan + threadIdx.x;  // j * dm + c
  if (i < (int64_t)M * dm) {
    // block order, as before; the unrolling only keeps 8 loads in flight
    float s = 0.f;
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(b + u) * M * dm + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < nblk; ++b) s += part[(int64_t)b * M * dm + i];
    dWr[i] = s;
  }
  if (db && blockIdx.x == 0 && threadIdx.x < M) {
    float s = 0.f;
    for (int b = 0; b < nblk; ++b) s += dbp[(int64_t)b * M + threadIdx.x];
    db[threadIdx.x] = s;
  }
}

template <int MB>
void launch_router_bwd(const float* dl, const uint16_t* X, const uint16_t* Wr, int64_t N, int dm, int M, float* dX,
                       float* dWr, float* db, float* part, float* dbp, int nblk, hipStream_t st) {
  const unsigned cblk = (unsigned)ceil_div(dm, kChan);
  router_dx_kernel<MB><<<dim3((unsigned)ceil_div(N, kDxTokens), cblk), kChan, 0, st>>>(dl, Wr, N, dm, M, dX);
  const unsigned wblk = (unsigned)ceil_div(dm, kChan * dw_cpt<MB>());
  router_dw_partial_kernel<MB><<<dim3((unsigned)nblk, wblk), kChan, 0, st>>>(dl, X, N, dm, M, part, dbp);
  router_dw_reduce_kernel<<<(unsigned)ceil_div((int64_t)M * dm, kChan), kChan, 0, st>>>(part, dbp, nblk, dm, M, dWr,
                                                                                       db);
}

}  // namespace
}  // namespace moga

extern "C" int moga_unpermute_backward(const void* dO, const void* Op, const int32_t* perm, const float* gate,
                                       int64_t N, int32_t H, int32_t D, void* dOp, float* delta, float* dgate,
                                       void* stream) {
  using namespace moga;
  if (!dO || !Op || !perm || !gate || !dOp || !delta || !dgate) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || H < 1 || D < 1) return MOGA_ERR_SHAPE;
  if (!valid_head_dims(H, D)) return MOGA_ERR_UNSUPPORTED;
  hipStream_t st = as_stream(stream);
  unpermute_backward_kernel<<<dim3((unsigned)ceil_div(N, kUbWaves)), kUbWaves * kWave, 0, st>>>(
      static_cast<const uint16_t*>(dO), static_cast<const uint16_t*>(Op), perm, gate, N, H, D,
      static_cast<uint16_t*>(dOp), delta, dgate);
  MOGA_LAUNCH_CHECK();
  return MOGA_OK;
}

extern "C" int moga_route_backward(const void* X, const void* Wr, const float* bias, const int32_t* group_id,
                                   const float* dgate, int64_t N, int32_t d_model, int32_t M, float* dX, float* dWr,
                                   float* dbias, void* ws, size_t ws_bytes, void* stream) {
  using namespace moga;
  if (!X || !Wr || !group_id || !dgate || !dX || !dWr) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1 || d_model < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups || d_model % 32 != 0) return MOGA_ERR_UNSUPPORTED;
  const size_t need = moga_workspace_bytes(MOGA_OP_ROUTE_BACKWARD, N, M, 1, d_model);
  if (!ws || ws_bytes < need) return MOGA_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  const auto* x = static_cast<const uint16_t*>(X);
  const auto* w = static_cast<const uint16_t*>(Wr);
  const int nblk = (int)ceil_div(N, kDwTokens);
  char* p = static_cast<char*>(ws);
  float* dl = reinterpret_cast<float*>(p);
  p += align_up((size_t)N * M * 4, 256);
  float* part = reinterpret_cast<float*>(p);
  p += align_up((size_t)nblk * M * d_model * 4, 256);
  float* dbp = reinterpret_cast<float*>(p);
  const int rc = moga_route_dlogits(x, w, bias, N, d_model, M, group_id, dgate, dl, st);
  if (rc != MOGA_OK) return rc;
  switch ((M + 15) / 16) {
    case 1: launch_router_bwd<1>(dl, x, w, N, d_model, M, dX, dWr, dbias, part, dbp, nblk, st); break;
    case 2: launch_router_bwd<2>(dl, x, w, N, d_model, M, dX, dWr, dbias, part, dbp, nblk, st); break;
    case 3: launch_router_bwd<3>(dl, x, w, N, d_model, M, dX, dWr, dbias, part, dbp, nblk, st); break;
    default: launch_router_bwd<4>(dl, x, w, N, d_model, M, dX, dWr, dbias, part, dbp, nblk, st); break;
  }
  MOGA_LAUNCH_CHECK();
  return MOGA_OK;
}
