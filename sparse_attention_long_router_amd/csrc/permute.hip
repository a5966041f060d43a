// Group permutation: stable counting sort of tokens by group id, then a
// row gather of Q, K, V into group-contiguous order.
// Page "MoGA: Mixture-of-Groups Attention for End-to-End Long Video
// Generation", section "MoGA Pseudocode and Kernel Integration", Algorithm 1
// step 2 (group 0 first, then group 1, ...; cu_seqlen, max_seqlen and the
// permute index as by-products).
//
// Four launches on the caller's stream, no host round trip:
//   hist_kernel     per 1024-token block, count tokens of each group (LDS)
//   scan_kernel     one workgroup: exclusive scan of the [M][blocks] counts in
//                   group-major order -> each (group, block) base offset,
//                   cu_seqlens and max_seqlen
//   scatter_kernel  per block, stable ranks from wave ballots: lanes holding
//                   the same group id find each other with log2(M) ballots,
//                   rank = popcount of lower matching lanes; waves of a round
//                   are ordered through LDS counts -> perm[base + rank] = n
//   gather_kernel   Qp/Kp/Vp[j] = Q/K/V[perm[j]], whole H*D rows, 16-byte
//                   lanes, one wave per row copy (HBM-bound stream)
// moga_permute_vt runs the same sort, gathers only Q and K as rows (or K
// alone, for an attention that reads Q through perm) and writes V transposed
// per head (gather_vt_kernel): Vt[h][d][j], the layout whose 64-key tiles the
// attention reads with one 16-byte LDS read per MFMA operand.
#include <mutex>

#include "moga_internal.h"

// Sort scratch of moga_permute_vt_noalloc (the [M][blocks] counts and base
// offsets of the counting sort): a fixed device array, one copy per GPU,
// held until the process ends.  In host code `scratch` only names the symbol;
// its device address comes from hipGetSymbolAddress (scratch_address below).
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;  // 1 MiB
static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

namespace moga {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / kWave;

__global__ __launch_bounds__(kSortThreads) void hist_kernel(const int32_t* __restrict__ gid, int64_t N, int M,
                                                          int nblk, int32_t* __restrict__ hist) {
  __shared__ int h[kMaxGroups];
  if (threadIdx.x < kMaxGroups) h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t n0 = (int64_t)blockIdx.x * kSortChunk;
  for (int i = threadIdx.x; i < kSortChunk; i += kSortThreads) {
    const int64_t n = n0 + i;
    if (n < N) atomicAdd(&h[gid[n]], 1);
  }
  __syncthreads();
  if (threadIdx.x < M) hist[(int64_t)threadIdx.x * nblk + blockIdx.x] = h[threadIdx.x];
}

constexpr int kScanThreads = 1024;

// Exclusive scan over E = M * nblk counts laid out group-major.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ hist, int M, int nblk,
                                                          int64_t N, int32_t* __restrict__ base,
                                                          int32_t* __restrict__ cu, int32_t* __restrict__ max_seqlen) {
  __shared__ int part[kScanThreads];
  const int64_t E = (int64_t)M * nblk;
  const int64_t per = (E + kScanThreads - 1) / kScanThreads;
  const int64_t lo = threadIdx.x * per;
  const int64_t hi = lo + per < E ? lo + per : E;
  int s = 0;
  for (int64_t e = lo; e < hi; ++e) s += hist[e];
  part[threadIdx.x] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan of the per-thread sums
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = threadIdx.x ? part[threadIdx.x - 1] : 0;
  for (int64_t e = lo; e < hi; ++e) {
    base[e] = run;
    if (e % nblk == 0) cu[e / nblk] = run;  // first block of group e / nblk
    run += hist[e];
  }
  if (threadIdx.x == 0) cu[M] = (int32_t)N;
  __syncthreads();  // makes every cu entry visible to the block
  if (threadIdx.x < kWave) {  // max group size over M <= 64 entries: wave 0 only
    int v = 0;
    if (threadIdx.x < M) v = cu[threadIdx.x + 1] - cu[threadIdx.x];
    for (int off = 32; off >= 1; off >>= 1) {
      const int o = __shfl_xor(v, off);
      v = o > v ? o : v;
    }
    if (threadIdx.x == 0) *max_seqlen = v;
  }
}

__global__ __launch_bounds__(kSortThreads) void scatter_kernel(const int32_t* __restrict__ gid, int64_t N, int M,
                                                             int nblk, const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ perm) {
  __shared__ int run[kMaxGroups];
  __shared__ int wcnt[kSortWaves][kMaxGroups];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x < M) run[threadIdx.x] = base[(int64_t)threadIdx.x * nblk + blockIdx.x];
  for (int i = threadIdx.x; i < kSortWaves * kMaxGroups; i += kSortThreads) (&wcnt[0][0])[i] = 0;
  int bits = 0;
  while ((1 << bits) < M) ++bits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  __syncthreads();

  const int64_t n0 = (int64_t)blockIdx.x * kSortChunk;
  for (int r0 = 0; r0 < kSortChunk; r0 += kSortThreads) {
    const int64_t n = n0 + r0 + threadIdx.x;
    const bool valid = n < N;
    const int g = valid ? gid[n] : 0;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (g >> b) & 1;
      const uint64_t ones = __ballot(valid && bit);
      match &= bit ? ones : ~ones;
    }
    const int rank = __popcll(match & lt_mask);
    if (valid && rank == 0) wcnt[wave][g] = __popcll(match);
    __syncthreads();
    if (valid) {
      int off = run[g] + rank;
      for (int w = 0; w < wave; ++w) off += wcnt[w][g];
      perm[off] = (int32_t)n;
    }
    __syncthreads();
    if (threadIdx.x < M) {
      int add = 0;
      for (int w = 0; w < kSortWaves; ++w) {
        add += wcnt[w][threadIdx.x];
        wcnt[w][threadIdx.x] = 0;
      }
      run[threadIdx.x] += add;
    }
    __syncthreads();
  }
}

constexpr int kGatherWaves = 4;  // one token row per wave
constexpr int kGatherBatch = 3;  // 64-lane chunk steps loaded before any store

// Qp/Kp/Vp[j] = Q/K/V[perm[j]]; rows are `chunks` 16-byte pieces long.  Each
// wave copies one row of each tensor; all loads of a batch (three 1 KB
// contiguous pieces per tensor, the whole row at H*D = 1536) are in flight
// before the first store, which measured 4% faster than interleaving them.
template <bool kWithQ, bool kWithV>
__global__ __launch_bounds__(kGatherWaves * kWave) void gather_kernel(
    const int32_t* __restrict__ perm, int64_t N, int chunks, const u32x4* __restrict__ Q,
    const u32x4* __restrict__ K, const u32x4* __restrict__ V, u32x4* __restrict__ Qp, u32x4* __restrict__ Kp,
    u32x4* __restrict__ Vp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j = (int64_t)blockIdx.x * kGatherWaves + wave;
  if (j >= N) return;
  const int64_t src = (int64_t)perm[j] * chunks, dst = j * chunks;
  for (int c0 = 0; c0 < chunks; c0 += kGatherBatch * kWave) {
    u32x4 a[kGatherBatch], b[kGatherBatch], d[kGatherBatch];
#pragma unroll
    for (int u = 0; u < kGatherBatch; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < chunks) {
        if constexpr (kWithQ) a[u] = __builtin_nontemporal_load(Q + src + c);
        b[u] = __builtin_nontemporal_load(K + src + c);
        if constexpr (kWithV) d[u] = __builtin_nontemporal_load(V + src + c);
      }
    }
#pragma unroll
    for (int u = 0; u < kGatherBatch; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < chunks) {
        if constexpr (kWithQ) __builtin_nontemporal_store(a[u], Qp + dst + c);
        __builtin_nontemporal_store(b[u], Kp + dst + c);
        if constexpr (kWithV) __builtin_nontemporal_store(d[u], Vp + dst + c);
      }
    }
  }
}

// Vt[h][d][j] = V[perm[j]][h][d] for j < N and 0 for N <= j < ldv: V in
// permuted order, transposed per head (one zero-padded row per channel).  A
// workgroup takes 64 consecutive permuted tokens of one head: it reads their
// D-channel slices (D*2 contiguous bytes each) into LDS and writes D rows of
// 64 tokens (128 contiguous bytes, eight lanes) back out.  The LDS row pitch
// of D + 2 elements (65 dwords at D = 128) moves each row one bank on, so the
// column reads of the transposition and the row writes are both free of bank
// conflicts.
constexpr int kVtTile = 64;
template <int D>
__global__ __launch_bounds__(256) void gather_vt_kernel(const int32_t* __restrict__ perm, int64_t N, int64_t ldv,
                                                        int H, const uint16_t* __restrict__ V,
                                                        uint16_t* __restrict__ Vt) {
  constexpr int kPitch = D + 2;  // elements
  constexpr int CPT = D / 8;     // 16-byte chunks per token slice
  __shared__ __attribute__((aligned(16))) uint32_t tile[kVtTile * kPitch / 2];
  const int h = blockIdx.y;
  const int64_t j0 = (int64_t)blockIdx.x * kVtTile;  // ldv is a multiple of 64: the tile lies inside the row
  for (int c = threadIdx.x; c < kVtTile * CPT; c += 256) {
    const int tok = c / CPT, ch = c % CPT;
    const int64_t j = j0 + tok;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j < N) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(V + ((int64_t)perm[j] * H + h) * D) + ch);
    uint32_t* row = tile + tok * (kPitch / 2) + ch * 4;
    row[0] = v[0];
    row[1] = v[1];
    row[2] = v[2];
    row[3] = v[3];
  }
  __syncthreads();
  const uint16_t* t16 = reinterpret_cast<const uint16_t*>(tile);
  // channel row d, tokens 8u .. 8u+7
  for (int c = threadIdx.x; c < D * (kVtTile / 8); c += 256) {
    const int d = c >> 3, u = c & 7;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)t16[(8 * u + 2 * i) * kPitch + d] | ((uint32_t)t16[(8 * u + 2 * i + 1) * kPitch + d] << 16);
    __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]},
                                reinterpret_cast<u32x4*>(Vt + ((int64_t)h * D + d) * ldv + j0 + 8 * u));
  }
}

}  // namespace
}  // namespace moga

extern "C" int moga_permute(const int32_t* group_id, const void* Q, const void* K, const void* V, int64_t N,
                            int32_t H, int32_t D, int32_t M, void* Qp, void* Kp, void* Vp, int32_t* perm,
                            int32_t* cu_seqlens, int32_t* max_seqlen, void* ws, size_t ws_bytes, void* stream) {
  using namespace moga;
  if (!group_id || !perm || !cu_seqlens || !max_seqlen) return MOGA_ERR_NULL;
  const bool any_rows = Q || K || V || Qp || Kp || Vp;
  const bool all_rows = Q && K && V && Qp && Kp && Vp;
  if (any_rows && !all_rows) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups) return MOGA_ERR_UNSUPPORTED;
  if (all_rows && !valid_head_dims(H, D)) return (H < 1 || D < 1) ? MOGA_ERR_SHAPE : MOGA_ERR_UNSUPPORTED;
  const size_t need = moga_workspace_bytes(MOGA_OP_PERMUTE, N, M, H, D);
  if (!ws || ws_bytes < need) return MOGA_ERR_WORKSPACE;

  hipStream_t st = as_stream(stream);
  const int nblk = (int)sort_blocks(N);
  int32_t* hist = static_cast<int32_t*>(ws);
  int32_t* base = hist + (size_t)M * nblk;
  hist_kernel<<<nblk, kSortThreads, 0, st>>>(group_id, N, M, nblk, hist);
  MOGA_LAUNCH_CHECK();
  scan_kernel<<<1, kScanThreads, 0, st>>>(hist, M, nblk, N, base, cu_seqlens, max_seqlen);
  MOGA_LAUNCH_CHECK();
  scatter_kernel<<<nblk, kSortThreads, 0, st>>>(group_id, N, M, nblk, base, perm);
  MOGA_LAUNCH_CHECK();
  if (all_rows) {
    const int chunks = H * D / 8;
    const int64_t blocks = ceil_div(N, kGatherWaves);
    gather_kernel<true, true><<<dim3((unsigned)blocks), kGatherWaves * kWave, 0, st>>>(
        perm, N, chunks, static_cast<const u32x4*>(Q), static_cast<const u32x4*>(K), static_cast<const u32x4*>(V),
        static_cast<u32x4*>(Qp), static_cast<u32x4*>(Kp), static_cast<u32x4*>(Vp));
    MOGA_LAUNCH_CHECK();
  }
  return MOGA_OK;
}

namespace moga {
namespace {
int permute_vt_args(const int32_t* group_id, const void* Q, const void* K, const void* V, int64_t N, int32_t H,
                    int32_t D, int32_t M, const void* Qp, const void* Kp, const void* Vt, const int32_t* perm,
                    const int32_t* cu_seqlens, const int32_t* max_seqlen) {
  if (!group_id || !perm || !cu_seqlens || !max_seqlen || !K || !V || !Kp || !Vt) return MOGA_ERR_NULL;
  if (!Q != !Qp) return MOGA_ERR_NULL;  // Q is gathered only when both are given
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1 || H < 1 || D < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups || !valid_head_dims(H, D) || N > kVtMaxTokens) return MOGA_ERR_UNSUPPORTED;
  return MOGA_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept for the process.
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return MOGA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOGA_ERR_HIP;
    }
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MOGA_OK;
}
}  // namespace
}  // namespace moga

extern "C" int moga_permute_vt(const int32_t* group_id, const void* Q, const void* K, const void* V, int64_t N,
                               int32_t H, int32_t D, int32_t M, void* Qp, void* Kp, void* Vt, int32_t* perm,
                               int32_t* cu_seqlens, int32_t* max_seqlen, void* ws, size_t ws_bytes, void* stream) {
  using namespace moga;
  const int arg = permute_vt_args(group_id, Q, K, V, N, H, D, M, Qp, Kp, Vt, perm, cu_seqlens, max_seqlen);
  if (arg != MOGA_OK) return arg;
  // the sort, as moga_permute without row copies
  const int rc = moga_permute(group_id, nullptr, nullptr, nullptr, N, H, D, M, nullptr, nullptr, nullptr, perm,
                              cu_seqlens, max_seqlen, ws, ws_bytes, stream);
  if (rc != MOGA_OK) return rc;
  hipStream_t st = as_stream(stream);
  const int chunks = H * D / 8;
  const dim3 rows_grid((unsigned)ceil_div(N, kGatherWaves));
  if (Q)
    gather_kernel<true, false><<<rows_grid, kGatherWaves * kWave, 0, st>>>(
        perm, N, chunks, static_cast<const u32x4*>(Q), static_cast<const u32x4*>(K), nullptr,
        static_cast<u32x4*>(Qp), static_cast<u32x4*>(Kp), nullptr);
  else
    gather_kernel<false, false><<<rows_grid, kGatherWaves * kWave, 0, st>>>(
        perm, N, chunks, nullptr, static_cast<const u32x4*>(K), nullptr, nullptr, static_cast<u32x4*>(Kp), nullptr);
  MOGA_LAUNCH_CHECK();
  const int64_t ldv = vt_row_length(N);
  const dim3 grid((unsigned)(ldv / kVtTile), (unsigned)H);
  if (D == 128)
    gather_vt_kernel<128><<<grid, 256, 0, st>>>(perm, N, ldv, H, static_cast<const uint16_t*>(V),
                                               static_cast<uint16_t*>(Vt));
  else
    gather_vt_kernel<64><<<grid, 256, 0, st>>>(perm, N, ldv, H, static_cast<const uint16_t*>(V),
                                              static_cast<uint16_t*>(Vt));
  MOGA_LAUNCH_CHECK();
  return MOGA_OK;
}

extern "C" int moga_permute_vt_noalloc(const int32_t* group_id, const void* Q, const void* K, const void* V,
                                       int64_t N, int32_t H, int32_t D, int32_t M, void* Qp, void* Kp, void* Vt,
                                       int32_t* perm, int32_t* cu_seqlens, int32_t* max_seqlen, void* stream) {
  using namespace moga;
  const int arg = permute_vt_args(group_id, Q, K, V, N, H, D, M, Qp, Kp, Vt, perm, cu_seqlens, max_seqlen);
  if (arg != MOGA_OK) return arg;
  if (moga_workspace_bytes(MOGA_OP_PERMUTE, N, M, H, D) > kNoAllocScratchBytes) return MOGA_ERR_WORKSPACE;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != MOGA_OK) return rc;
  return moga_permute_vt(group_id, Q, K, V, N, H, D, M, Qp, Kp, Vt, perm, cu_seqlens, max_seqlen, ws,
                         kNoAllocScratchBytes, stream);
}
