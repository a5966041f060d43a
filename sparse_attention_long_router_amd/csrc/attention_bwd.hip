// Backward of the group attention for gfx950 (learned groups, permuted rows).
// Page "MoGA: Mixture-of-Groups Attention for End-to-End Long Video
// Generation": Eq. 1 restricted to a group (the MoGA output equation,
// "Grouped Attention"), differentiated with the softmax saved as its
// per-row log-sum-exp.  For a group and head, with c = scale:
//   P = exp(c Q K^T - lse),  dV = P^T dA,  dP = dA V^T,
//   dS = P * (dP - delta),   dQ = c dS K,  dK = c dS^T Q,
// where dA is the gated upstream gradient in permuted order and delta the
// row sums of dA * A (both from moga_unpermute_backward).
//
// Two kernels, a third for the staged form below; no atomics (results are
// bitwise repeatable):
//   dkdv_kernel: K and V rows of 32 keys per wave stay in registers as MFMA
//     operands; the group's queries stream through LDS in tiles of 128 (Q,
//     dA, lse, delta).  S = Q K^T puts one key per lane, so P and dS feed
//     dV^T += dA^T P and dK^T += Q^T dS directly as MFMA B operands, with
//     dA^T and Q^T read from LDS by transposing reads.
//   dq_kernel: Q and dA rows of 32 queries per wave stay in registers; keys
//     and values stream through LDS as in the forward pass.  S^T = K Q^T and
//     dP^T = V dA^T put one query per lane, and dQ^T += K^T dS^T.
// With a workspace large enough for it (moga_group_attention_backward decides
// on the device, head by head), dkdv_kernel also stores dS in bf16, which the
// dq kernel rounds it to anyway, and dq_ds_kernel computes dQ = c dS K from
// it: five products per group and head instead of seven (S and dP are not
// computed a second time), for sum_g n_g^2 * 2 bytes of HBM per staged head.
// The first Hs heads that fit are staged; dq_kernel takes the others.  The
// dS of group g, head h is stored in blocks of 32 queries x 32 keys (2 KB):
// block (qb, kb) at off[g] + ((h * nb + qb) * nbp + kb) * 2048 bytes, with
// nb = ceil(n_g / 32),
// nbp = nb rounded up to even (the padding block holds zeros).  A block is
// two 1 KB halves u = 0, 1, each 64 chunks of 16 bytes, chunk L = the 8
// queries at positions 16u + 8(L/32) .. 16u + 8(L/32) + 7 of key L%32, so
// that each of dkdv's two stores per block writes 1 KB in whole lines;
// position p stands for query p with bits 2 and 3 exchanged (the order of
// the dkdv MFMA result).
// Rows past a group's end are read as zeros through the buffer range check:
// a zero query row has a zero upstream gradient and a zero key row a zero
// operand, so they add nothing to the rows that are stored, and the exact
// P = exp(s - lse) needs no normaliser.  The dq kernel clamps the exponent
// at 2^0.5 (a valid key's weight is at most 1), so that a very negative
// log-sum-exp cannot turn the zero key rows of a group's last tile into
// inf * 0.
#include <stddef.h>

#include <type_traits>

#include "moga_internal.h"

typedef int32_t i32x4v __attribute__((ext_vector_type(4)));
__device__ void raw_buffer_load_lds(i32x4v rsrc, __attribute__((address_space(3))) void* lds, int size, int voffset,
                                    int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
// 16-byte raw buffer load into registers (offsets past the range read zeros)
// and store (stores past the range are dropped).
__device__ moga::u32x4 raw_buffer_load_x4(i32x4v rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ void raw_buffer_store_x4(moga::u32x4 data, i32x4v rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.store.v4i32");

namespace moga {
namespace {

constexpr int kTileQ = 128;    // query rows per streamed LDS tile (dkdv_kernel)
constexpr int kTileK = 128;    // key rows per streamed LDS tile (dq_kernel)
constexpr int kDqBM = 256;     // queries per dq work item (8 waves x 32)
constexpr int kDqWaves = 8;
constexpr int kDkvBN = 128;    // keys per dkdv work item (4 waves x 32)
constexpr int kDkvWaves = 4;
constexpr int kRun = 32;       // consecutive items per XCD, one per CU: about half the HBM reads of 8
constexpr int kDsTile = 64;    // keys per streamed LDS tile (dq_ds_kernel): two 32-key dS blocks
constexpr int kDsBlock = 2048; // bytes of one 32 x 32 dS block
constexpr int kCpolNt = 2;     // cache policy of the dS stores and loads: non-temporal, each byte is moved once

// Where the staged dS of each group starts, and how many heads fit the workspace.
struct DsPlan {
  int64_t off[kMaxGroups];  // byte offset of group g's blocks in the dS area
  int32_t heads;            // heads 0 .. heads-1 are staged: dkdv stores their dS, dq_ds_kernel forms their dQ
};
constexpr size_t kDsPlanOffset = 2048;  // in the workspace, after the two schedules
constexpr size_t kDsDataOffset = 4096;  // start of the dS area
static_assert(kDsPlanOffset + offsetof(DsPlan, heads) == MOGA_BWD_STAGED_FLAG_OFFSET, "flag offset in moga.h");
static_assert(kDsPlanOffset + sizeof(DsPlan) <= kDsDataOffset, "plan fits before the dS area");

__device__ __forceinline__ i32x4v byte_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  bytes = bytes < 0 ? 0 : (bytes < 0xffffffffll ? bytes : 0xffffffffll);
  i32x4v r;
  r[0] = (int32_t)(uint32_t)a;
  r[1] = (int32_t)(uint32_t)(a >> 32);
  r[2] = (int32_t)(uint32_t)bytes;
  r[3] = 0x00020000;
  return r;
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// 16-byte chunk swizzles (cpr = chunks per row): kRowsOnly keeps row reads
// conflict-free; kBoth keeps both row reads and transposing reads free of
// bank conflicts (distinct chunks for any 8 consecutive rows, and for the 4
// rows x 2 chunks of one transposing read group).
enum { kRowsOnly = 0, kBoth = 1 };
template <int kSwz>
__device__ __forceinline__ int swz(int r, int cpr) {
  if constexpr (kSwz == kRowsOnly) return r & (cpr - 1);
  return cpr == 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : (((r & 3) << 1) | ((r >> 2) & 1));
}

__device__ __forceinline__ i32x4v row_rsrc(const uint16_t* base, int64_t n_rows, int64_t row_bytes, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  int64_t range = n_rows > 0 ? (n_rows - 1) * row_bytes + bytes : 0;
  range = range < 0xffffffffll ? range : 0xffffffffll;
  i32x4v r;
  r[0] = (int32_t)(uint32_t)a;
  r[1] = (int32_t)(uint32_t)(a >> 32);
  r[2] = (int32_t)(uint32_t)range;
  r[3] = 0x00020000;
  return r;
}

// kTile rows of one head (row stride row_stride elements) into LDS, swizzled.
template <int D, int NW, int kSwz, int kTile>
__device__ __forceinline__ void load_tile(i32x4v rs, uint16_t* T, int64_t row_stride, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int LOADS = kTile * CPR / (NW * kWave);
  static_assert(LOADS >= 1 && kTile * CPR == LOADS * NW * kWave, "tile must split evenly over the waves");
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int q = (wave * LOADS + j) * kWave + lane;
    const int r = q / CPR, p = q % CPR;
    const int lds_off = (wave * LOADS + j) * kWave * 8;
    raw_buffer_load_lds(rs, (lds_void*)(T + lds_off), 16, r * (int)row_stride * 2 + ((p ^ swz<kSwz>(r, CPR)) << 4),
                        0, 0, 0);
  }
}

// A from 32 LDS rows (rbase..rbase+31), B from registers: C[m = row][n = lane % 32].
// Reg r of the result is row 8*(r/4) + 4*hh + r%4 of the block.
// c0 is the accumulator's starting value (zeros, or a per-row offset).
template <int D, int kSwz>
__device__ __forceinline__ f32x16 rows_mma(const uint16_t* T, int rbase, const bf16x8 (&b)[D / 16], int lane,
                                           f32x16 c0 = f32x16{}) {
  constexpr int CPR = D / 8;
  const int hh = lane >> 5, row = rbase + (lane & 31);
  bf16x8 a[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    a[st] = *reinterpret_cast<const bf16x8*>(T + row * D + ((2 * st + hh) ^ swz<kSwz>(row, CPR)) * 8);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 c = c0;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[st], b[st], c, 0, 0, 0);
  return c;
}

// rows_mma with the first half of the A operands read ahead and the rest just
// before their MFMAs.  The dq kernel keeps Q and dA fragments, the dQ
// accumulators and -delta live: reading all eight operands ahead needs 32 more
// VGPRs than it has and spills, reading each one just in time exposes an LDS
// round trip per MFMA (dq 30.3 ms; this form 29.5 ms, same box), and the
// second wave on the SIMD covers what latency is left.
template <int D, int kSwz>
__device__ __forceinline__ f32x16 rows_mma_half(const uint16_t* T, int rbase, const bf16x8 (&b)[D / 16], int lane,
                                                f32x16 c0 = f32x16{}) {
  constexpr int CPR = D / 8;
  constexpr int H2 = D / 32;
  const int hh = lane >> 5, row = rbase + (lane & 31);
  bf16x8 a[H2];
#pragma unroll
  for (int st = 0; st < H2; ++st)
    a[st] = *reinterpret_cast<const bf16x8*>(T + row * D + ((2 * st + hh) ^ swz<kSwz>(row, CPR)) * 8);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 c = c0;
#pragma unroll
  for (int st = 0; st < H2; ++st) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[st], b[st], c, 0, 0, 0);
#pragma unroll
  for (int st = H2; st < D / 16; ++st)
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        *reinterpret_cast<const bf16x8*>(T + row * D + ((2 * st + hh) ^ swz<kSwz>(row, CPR)) * 8), b[st], c, 0, 0, 0);
  return c;
}

// acc[db] (C = T^T block: 32 channels x 32 columns) += T[rows]^T * p over the
// 32 LDS rows rbase..rbase+31, with A = T^T from transposing reads and
// B = p, whose k-slots follow the C layout of rows_mma (reg 8t + j of the
// half is row 16t + 8*(j/4) + 4*hh + j%4).
// kOneOffset: each address is one offset from T, so that the compiler can
// name the LDS array a read touches and not wait for loads into the others.
template <int D, int kSwz, bool kOneOffset = false>
__device__ __forceinline__ void tr_mma(const uint16_t* T, int rbase, const bf16x8 (&p)[2], int lane,
                                       f32x16 (&acc)[D / 32]) {
  constexpr int CPR = D / 8;
  const int hh = lane >> 5;
  const int tr_r = (lane & 15) >> 2, tr_q = lane & 3, tr_g = (lane >> 4) & 1;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r1 = rbase + 16 * t + 4 * hh + tr_r;
    const int r2 = r1 + 8;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = 32 * db + 16 * tr_g + 4 * tr_q;
      const int ch = col >> 3, within = col & 7;
      i16x4 lo, hi;
      if constexpr (kOneOffset) {
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(T + (r1 * D + ((ch ^ swz<kSwz>(r1, CPR)) << 3) + within)));
        hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(T + (r2 * D + ((ch ^ swz<kSwz>(r2, CPR)) << 3) + within)));
      } else {
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(T + r1 * D + ((ch ^ swz<kSwz>(r1, CPR)) << 3) + within));
        hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(T + r2 * D + ((ch ^ swz<kSwz>(r2, CPR)) << 3) + within));
      }
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[t], acc[db], 0, 0, 0);
    }
  }
}

// MFMA B-operand fragments of one row (lane % 32 picks the row, lane / 32 the
// 8-channel half of each 16-channel step); zeros past n_rows.
template <int D>
__device__ __forceinline__ void load_frags(const uint16_t* __restrict__ base, int64_t row_stride, int row, int n_rows,
                                           int lane, bf16x8 (&f)[D / 16]) {
  const int hh = lane >> 5;
  if (row < n_rows) {
    const uint16_t* p = base + (int64_t)row * row_stride + 8 * hh;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) f[st] = *reinterpret_cast<const bf16x8*>(p + 16 * st);
  } else {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) f[st] = bf16x8{};
  }
}

// Store a C-layout accumulator (lane = row of the output, reg r of block db =
// channel 32*db + 8*(r/4) + 4*hh + r%4) times s as bf16 to out[orow].
template <int D>
__device__ __forceinline__ void store_rows(uint16_t* __restrict__ out, const f32x16 (&acc)[D / 32], float s, int hh) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * db + 8 * q4 + 4 * hh;
      const u32x2 pk = {pack_bf16x2(acc[db][4 * q4] * s, acc[db][4 * q4 + 1] * s),
                        pack_bf16x2(acc[db][4 * q4 + 2] * s, acc[db][4 * q4 + 3] * s)};
      *reinterpret_cast<u32x2*>(out + d0) = pk;
    }
}

struct Item {
  int len;     // group size
  int t0;      // first row (group-local) of this item
  int head;
  int row0;    // first permuted row of the group
  int g;       // group index
};

__device__ __forceinline__ bool decode(const AttnSchedule* sched, const int32_t* cu, int M, int tile, int item,
                                       Item& w) {
  if (item >= sched->prefix[M]) return false;
  int i = 0;
  while (i + 1 < M && sched->prefix[i + 1] <= item) ++i;
  const int g = sched->order[i];
  const int local = item - sched->prefix[i];
  w.g = g;
  w.row0 = cu[g];
  w.len = cu[g + 1] - w.row0;
  const int nt = (w.len + tile - 1) / tile;
  w.head = local / nt;
  w.t0 = (local - w.head * nt) * tile;
  return true;
}

// ---------------------------------------------------------------------------
// dK, dV: 4 waves x 32 keys, queries streamed in tiles of kTileQ (128)
// kStage: the kernel may stage dS (the plan names the heads).
// ---------------------------------------------------------------------------
// One dkdv work item; kStage: this head's dS is staged (also stored).
template <int D, bool kStage>
__device__ __forceinline__ void dkdv_item(
    const Item& w, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dA, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ perm, int64_t N, int64_t row_stride, float scale, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, const DsPlan* __restrict__ plan, uint8_t* __restrict__ ds,
    uint16_t (&Qs)[2][kTileQ * D], uint16_t (&As)[2][kTileQ * D], float (&Ls)[2][kTileQ], float (&Ds)[2][kTileQ]) {
  constexpr int DBLK = D / 32;
  constexpr int NW = kDkvWaves;
  constexpr int kTile = kTileQ;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar descriptors, no waterfall
  const int64_t hoff = (int64_t)w.head * D;
  const int ntiles = (w.len + kTile - 1) / kTile;
  const float c2 = scale * 1.4426950408889634f;  // scores to log2 units

  // tile t: Q and dA rows, lse and delta of queries t*kTile .. t*kTile+kTile-1
  auto issue = [&](int buf, int t) {
    const int64_t first = (int64_t)w.row0 + (int64_t)t * kTile;
    const int64_t n = w.len - (int64_t)t * kTile;
    load_tile<D, NW, kBoth, kTile>(row_rsrc(Q + first * row_stride + hoff, n, row_stride * 2, D * 2), Qs[buf], row_stride,
                            wave, lane);
    load_tile<D, NW, kBoth, kTile>(row_rsrc(dA + first * row_stride + hoff, n, row_stride * 2, D * 2), As[buf], row_stride,
                            wave, lane);
    if (wave < kTile / kWave) {  // 64 entries per wave; past the group end the range is empty
      const int o = wave * kWave;
      const float* lp = lse + (int64_t)w.head * N + first + o;
      const float* dp = delta + (int64_t)w.head * N + first + o;
      raw_buffer_load_lds(row_rsrc(reinterpret_cast<const uint16_t*>(lp), n - o, 4, 4), (lds_void*)(Ls[buf] + o), 4,
                          lane * 4, 0, 0, 0);
      raw_buffer_load_lds(row_rsrc(reinterpret_cast<const uint16_t*>(dp), n - o, 4, 4), (lds_void*)(Ds[buf] + o), 4,
                          lane * 4, 0, 0, 0);
    }
  };
  issue(0, 0);

  // this wave's 32 keys as B operands (zeros past the group end)
  const int key = w.t0 + wave * 32 + (lane & 31);
  bf16x8 kf[D / 16], vf[D / 16];
  load_frags<D>(K + (int64_t)w.row0 * row_stride + hoff, row_stride, key, w.len, lane, kf);
  load_frags<D>(V + (int64_t)w.row0 * row_stride + hoff, row_stride, key, w.len, lane, vf);

  f32x16 dk[DBLK], dv[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // Staged dS: this wave's column of 32-key blocks.  The stores go through a
  // buffer descriptor per tile whose range ends after the group's last query
  // block (empty when nothing is staged), so that blocks past it are dropped
  // by the range check: no branch splits the block's MFMA and LDS stream.
  const uint8_t* ds_col = ds;  // block (0, kblk) of this wave's column
  int ds_nb = 0;               // query blocks of the group (0: nothing staged)
  uint32_t ds_pitch = 0;       // bytes between query blocks of the column
  if constexpr (kStage) {
    const int nb = (w.len + 31) >> 5, nbp = (nb + 1) & ~1;
    const int kblk = (w.t0 >> 5) + wave;  // uniform per wave
    if (kblk < nbp) {
      ds_col = ds + plan->off[w.g] + ((int64_t)w.head * nb * nbp + kblk) * kDsBlock;
      ds_nb = nb;
      ds_pitch = (uint32_t)nbp * kDsBlock;
    }
  }

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    __builtin_amdgcn_s_waitcnt(0);
    if (wave < kTile / kWave) {
      // This wave's lse and delta entries of the tile have landed: turn them
      // into the forms the loop consumes, lse in log2 units and -delta (the
      // starting value of the dP accumulator, so that it yields dP - delta).
      const int o = wave * kWave + lane;
      Ls[buf][o] *= 1.4426950408889634f;
      Ds[buf][o] = -Ds[buf][o];
    }
    __syncthreads();
    if (t + 1 < ntiles) issue(buf ^ 1, t + 1);
    const uint16_t* Qt = Qs[buf];
    const uint16_t* At = As[buf];
    i32x4v srs{};
    if constexpr (kStage) {
      // query blocks t*kQB .. of this wave's column that the group has
      const int rows = ds_nb - t * (kTile / 32);
      const int rc = rows < kTile / 32 ? rows : kTile / 32;
      srs = byte_rsrc(ds_col + (int64_t)t * (kTile / 32) * ds_pitch,
                      rc > 0 ? (int64_t)(rc - 1) * ds_pitch + kDsBlock : 0);
    }
#pragma unroll
    for (int qb = 0; qb < kTile / 32; ++qb) {
      // reg r of a C-layout block is row qb*32 + 8*(r/4) + 4*hh + r%4
      f32x16 nd;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Ds[buf][qb * 32 + 8 * g + 4 * hh]);
#pragma unroll
        for (int i = 0; i < 4; ++i) nd[4 * g + i] = d4[i];
      }
      const f32x16 s = rows_mma<D, kBoth>(Qt, qb * 32, kf, lane);       // S[query][key]
      const f32x16 dp = rows_mma<D, kBoth>(At, qb * 32, vf, lane, nd);  // dP[query][key] - delta[query]
      bf16x8 pb[2], sb[2];
      float pf[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&Ls[buf][qb * 32 + 8 * g + 4 * hh]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          pf[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -l4[i]));
          pb[r >> 3][r & 7] = (__bf16)pf[r];
        }
      }
      tr_mma<D, kBoth>(At, qb * 32, pb, lane, dv);  // dV^T += dA^T P
#pragma unroll
      for (int r = 0; r < 16; ++r) sb[r >> 3][r & 7] = (__bf16)(pf[r] * dp[r]);
      tr_mma<D, kBoth>(Qt, qb * 32, sb, lane, dk);  // dK^T += Q^T dS
      if constexpr (kStage) {
        // keys past the group end store zeros: their P has no bound
        const bool kv = key < w.len;
        const u32x4 z{};
        const u32x4 v0 = kv ? __builtin_bit_cast(u32x4, sb[0]) : z;
        const u32x4 v1 = kv ? __builtin_bit_cast(u32x4, sb[1]) : z;
        const int soff = (int)(qb * ds_pitch);
        raw_buffer_store_x4(v0, srs, lane * 16, soff, kCpolNt);
        raw_buffer_store_x4(v1, srs, lane * 16 + 1024, soff, kCpolNt);
      }
    }
  }

  if (key < w.len) {
    const int64_t orow = perm[w.row0 + key];
    store_rows<D>(dK + orow * row_stride + hoff, dk, scale, hh);
    store_rows<D>(dV + orow * row_stride + hoff, dv, 1.0f, hh);
  }
}

template <int D, bool kStage>
__global__ __launch_bounds__(kDkvWaves * kWave) void dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dA, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ perm, const AttnSchedule* __restrict__ sched, int M,
    int64_t N, int64_t row_stride, float scale, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    const DsPlan* __restrict__ plan, uint8_t* __restrict__ ds) {
  __shared__ __attribute__((aligned(1024))) uint16_t Qs[2][kTileQ * D];
  __shared__ __attribute__((aligned(1024))) uint16_t As[2][kTileQ * D];
  __shared__ __attribute__((aligned(256))) float Ls[2][kTileQ];
  __shared__ __attribute__((aligned(256))) float Ds[2][kTileQ];

  Item w;
  if (!decode(sched, cu, M, kDkvBN, xcd_remap(blockIdx.x, kRun), w)) return;
  if constexpr (kStage) {
    // heads past the plan's count run the form without stores
    if (w.head < plan->heads) {
      dkdv_item<D, true>(w, Q, K, V, dA, lse, delta, perm, N, row_stride, scale, dK, dV, plan, ds, Qs, As, Ls, Ds);
      return;
    }
  }
  dkdv_item<D, false>(w, Q, K, V, dA, lse, delta, perm, N, row_stride, scale, dK, dV, plan, ds, Qs, As, Ls, Ds);
}

// ---------------------------------------------------------------------------
// dQ: 8 waves x 32 queries, keys and values streamed in tiles of kTileK (128)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kDqWaves * kWave) void dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dA, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ perm, const AttnSchedule* __restrict__ sched, int M,
    int64_t N, int64_t row_stride, float scale, uint16_t* __restrict__ dQ, const DsPlan* __restrict__ plan) {
  constexpr int DBLK = D / 32;
  constexpr int NW = kDqWaves;
  constexpr int kTile = kTileK;
  __shared__ __attribute__((aligned(1024))) uint16_t Ks[2][kTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs[2][kTile * D];

  Item w;
  if (!decode(sched, cu, M, kDqBM, xcd_remap(blockIdx.x, kRun), w)) return;
  if (plan != nullptr && w.head < plan->heads) return;  // dq_ds_kernel forms this head's dQ from the staged dS
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t hoff = (int64_t)w.head * D;
  const int ntiles = (w.len + kTile - 1) / kTile;
  const float c2 = scale * 1.4426950408889634f;

  auto issue = [&](int buf, int t) {
    const int64_t first = (int64_t)w.row0 + (int64_t)t * kTile;
    const int64_t n = w.len - (int64_t)t * kTile;
    load_tile<D, NW, kBoth, kTile>(row_rsrc(K + first * row_stride + hoff, n, row_stride * 2, D * 2), Ks[buf], row_stride,
                            wave, lane);
    load_tile<D, NW, kRowsOnly, kTile>(row_rsrc(V + first * row_stride + hoff, n, row_stride * 2, D * 2), Vs[buf],
                                row_stride, wave, lane);
  };
  issue(0, 0);

  const int qi = w.t0 + wave * 32 + (lane & 31);
  bf16x8 qf[D / 16], af[D / 16];
  load_frags<D>(Q + (int64_t)w.row0 * row_stride + hoff, row_stride, qi, w.len, lane, qf);
  load_frags<D>(dA + (int64_t)w.row0 * row_stride + hoff, row_stride, qi, w.len, lane, af);
  const bool qvalid = qi < w.len;
  const float l2 = qvalid ? lse[(int64_t)w.head * N + w.row0 + qi] * 1.4426950408889634f : 0.f;
  const float dl = qvalid ? delta[(int64_t)w.head * N + w.row0 + qi] : 0.f;

  f32x16 dq[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) dq[db] = f32x16{};
  f32x16 ndl;  // -delta of this lane's query: the dP^T accumulator starts there and yields dP^T - delta
#pragma unroll
  for (int r = 0; r < 16; ++r) ndl[r] = -dl;

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles) issue(buf ^ 1, t + 1);
#pragma unroll
    for (int kb = 0; kb < kTile / 32; ++kb) {
      // S^T[key][query] and dP^T[key][query]; at D = 64 the preloading form
      // keeps three waves per SIMD, at D = 128 the half-preloading one fits
      f32x16 s, dp;
      if constexpr (D == 128) {
        s = rows_mma_half<D, kBoth>(Ks[buf], kb * 32, qf, lane);
        dp = rows_mma_half<D, kRowsOnly>(Vs[buf], kb * 32, af, lane, ndl);
      } else {
        s = rows_mma<D, kBoth>(Ks[buf], kb * 32, qf, lane);
        dp = rows_mma<D, kRowsOnly>(Vs[buf], kb * 32, af, lane, ndl);
      }
      bf16x8 sb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // A key of the group has s * c2 <= l2 (the log-sum-exp bounds every
        // term), so the exponent is at most a rounding error above 0 and the
        // clamp never binds.  The zero key rows past the group end have s = 0,
        // where a very negative log-sum-exp would overflow p and turn their
        // zero product into inf * 0; clamped, p stays finite and they add 0.
        const float p = __builtin_amdgcn_exp2f(fminf(fmaf(s[r], c2, -l2), 0.5f));
        sb[r >> 3][r & 7] = (__bf16)(p * dp[r]);
      }
      tr_mma<D, kBoth>(Ks[buf], kb * 32, sb, lane, dq);  // dQ^T += K^T dS^T
    }
  }

  if (qvalid) store_rows<D>(dQ + (int64_t)perm[w.row0 + qi] * row_stride + hoff, dq, scale, hh);
}

// ---------------------------------------------------------------------------
// dQ from the staged dS: 8 waves x 32 queries (one dS block row per wave),
// keys streamed in tiles of 64 (K rows shared, each wave's two dS blocks of
// its own).  The dS bytes come from HBM once each, so the stream runs two
// tiles ahead: tile t+2 is loaded into registers while tile t is used and
// tile t+1 waits in registers to be written to LDS at the end of tile t
// (register loads, whose waits the compiler counts exactly; it cannot tell
// LDS-DMA buffers apart across the loop).  dQ^T += K^T dS^T with both
// operands from transposing reads; the result's column n is the block
// position n, i.e. query n with bits 2 and 3 exchanged.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kDqWaves * kWave) void dq_ds_kernel(
    const uint16_t* __restrict__ K, const uint8_t* __restrict__ ds, const DsPlan* __restrict__ plan,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ perm, const AttnSchedule* __restrict__ sched, int M,
    int64_t row_stride, float scale, uint16_t* __restrict__ dQ) {
  constexpr int DBLK = D / 32;
  constexpr int NW = kDqWaves;
  constexpr int kT = kDsTile;
  constexpr int CPR = D / 8;
  constexpr int kSw = kT * 32;                        // elements of one wave's dS tile (64 key rows x 32 positions)
  constexpr int kLoadsK = kT * CPR / (NW * kWave);    // 16-byte K chunks per lane per tile
  constexpr int kLoadsS = kSw * 2 / (kWave * 16);     // 16-byte dS chunks per lane per tile
  static_assert(kLoadsK >= 1 && kLoadsK * NW * kWave == kT * CPR, "K tile splits evenly over the lanes");
  __shared__ __attribute__((aligned(1024))) uint16_t Kl0[kT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Kl1[kT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Sl0[NW * kSw];
  __shared__ __attribute__((aligned(1024))) uint16_t Sl1[NW * kSw];

  Item w;
  if (!decode(sched, cu, M, kDqBM, xcd_remap(blockIdx.x, kRun), w)) return;
  if (w.head >= plan->heads) return;  // dq_kernel computes this head's dQ
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t hoff = (int64_t)w.head * D;
  const int nb = (w.len + 31) >> 5, nbp = (nb + 1) & ~1;
  const int ntiles = nbp >> 1;
  const int qblk = (w.t0 >> 5) + wave;
  const bool live = qblk < nb;  // uniform per wave: the wave has queries of the group
  const i32x4v drs = byte_rsrc(ds + plan->off[w.g] + ((int64_t)w.head * nb + (live ? qblk : 0)) * nbp * kDsBlock,
                               live ? (int64_t)nbp * kDsBlock : 0);
  const int tr_r = (lane & 15) >> 2, tr_q = lane & 3, tr_g = (lane >> 4) & 1;

  // register staging of two tiles: slot 0 holds even tiles, slot 1 odd ones
  u32x4 rk[2][kLoadsK], rs[2][kLoadsS];
  auto load = [&](auto slotc, int t) __attribute__((always_inline)) {
    constexpr int sl = decltype(slotc)::value;
    const int64_t first = (int64_t)w.row0 + (int64_t)t * kT;
    const i32x4v krs = row_rsrc(K + first * row_stride + hoff, w.len - (int64_t)t * kT, row_stride * 2, D * 2);
#pragma unroll
    for (int j = 0; j < kLoadsK; ++j) {
      const int q = (wave * kLoadsK + j) * kWave + lane;
      const int r = q / CPR, c = q % CPR;
      rk[sl][j] = raw_buffer_load_x4(krs, r * (int)row_stride * 2 + c * 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kLoadsS; ++j)
      rs[sl][j] = raw_buffer_load_x4(drs, t * (2 * kDsBlock) + j * kWave * 16 + lane * 16, 0, kCpolNt);
  };
  // K chunk c of row r goes to LDS chunk c ^ swz(r) (the transposing reads'
  // swizzle); dS chunk L of the j-th KB (block j/2, half u = j%2) holds the
  // 8 positions 16u + 8(L/32) .. of key L%32, and goes to that key's row
  // (64 bytes) of the wave's LDS tile.
  auto store = [&](auto slotc, uint16_t* Kb, uint16_t* Sb) __attribute__((always_inline)) {
    constexpr int sl = decltype(slotc)::value;
#pragma unroll
    for (int j = 0; j < kLoadsK; ++j) {
      const int q = (wave * kLoadsK + j) * kWave + lane;
      const int r = q / CPR, c = q % CPR;
      *reinterpret_cast<u32x4*>(Kb + (r * D + ((c ^ swz<kBoth>(r, CPR)) << 3))) = rk[sl][j];
    }
#pragma unroll
    for (int j = 0; j < kLoadsS; ++j) {
      const int o = wave * kSw + (j >> 1) * 1024 + (lane & 31) * 32 + 16 * (j & 1) + 8 * (lane >> 5);
      *reinterpret_cast<u32x4*>(Sb + o) = rs[sl][j];
    }
  };
  // LDS writes done, then the barrier; the empty asm statements keep the
  // compiler from moving LDS accesses across it (s_barrier itself names no
  // memory).  A plain s_barrier: __syncthreads()'s fence would also wait for
  // the register loads in flight.
  auto sync = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16 acc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) acc[db] = f32x16{};

  auto compute = [&](const uint16_t* Kb, const uint16_t* Sb) __attribute__((always_inline)) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      bf16x8 b[2];  // dS^T operands of keys 32*h2 + 16*u + (k-slot rows), position = lane % 32
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r1 = 32 * h2 + 16 * u + 4 * hh + tr_r;
        const int o = wave * kSw + r1 * 32 + 16 * tr_g + 4 * tr_q;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Sb + o));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Sb + (o + 8 * 32)));
        b[u] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      tr_mma<D, kBoth>(Kb, 32 * h2, b, lane, acc);
    }
  };
  // tile t (parity P, LDS buffers P): barrier (tile t written by all waves),
  // load tile t+2 into register slot P (free: tile t left it for LDS at the
  // end of tile t-1), compute tile t, then write tile t+1 (slot 1-P, loaded
  // during tile t-1) into buffers 1-P, which tile t-1 finished reading
  // before the barrier.  Every wave issues the same loads and writes on
  // every tile (a wave without queries and the tiles past the last load
  // zeros through empty descriptor ranges), so that the compiler's counted
  // waits stay exact across the loop; tiles are taken in pairs, the one past
  // an odd count holding zeros only.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto tile = [&](auto par, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    uint16_t* Kb = P == 0 ? Kl0 : Kl1;
    uint16_t* Sb = P == 0 ? Sl0 : Sl1;
    uint16_t* Kn = P == 0 ? Kl1 : Kl0;
    uint16_t* Sn = P == 0 ? Sl1 : Sl0;
    sync();
    load(par, t + 2);
    if (live) compute(Kb, Sb);
    store(std::integral_constant<int, 1 - P>{}, Kn, Sn);
  };
  load(I0{}, 0);
  load(I1{}, 1);
  store(I0{}, Kl0, Sl0);
  for (int t = 0; t < ntiles; t += 2) {
    tile(I0{}, t);
    tile(I1{}, t + 1);
  }

  if (live) {
    const int p = lane & 31;
    const int qi = qblk * 32 + ((p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1));
    if (qi < w.len) store_rows<D>(dQ + (int64_t)perm[w.row0 + qi] * row_stride + hoff, acc, scale, hh);
  }
}

// Staged-dS plan: as many heads as the capacity holds (all of them, or the
// first Hs), and per-group byte offsets of their blocks (group index order,
// group g holding Hs * nb_g * nbp_g blocks).  One wave; a group's bytes per
// head saturate at 2^50 so that the sum cannot overflow (such a group never
// fits).
__global__ __launch_bounds__(kWave) void ds_plan_kernel(const int32_t* __restrict__ cu, int M, int H,
                                                      int64_t capacity, DsPlan* __restrict__ plan) {
  const int g = threadIdx.x;
  const int64_t cap = int64_t(1) << 50;
  int64_t bytes = 0;  // per head
  if (g < M) {
    const int64_t n = (int64_t)cu[g + 1] - cu[g];
    const int64_t nb = (n + 31) >> 5, nbp = (nb + 1) & ~int64_t(1);
    bytes = nb > (int64_t(1) << 19) ? cap : nb * nbp * kDsBlock;
  }
  int64_t incl = bytes;
  for (int off = 1; off < kWave; off <<= 1) {
    const int64_t v = __shfl_up(incl, off);
    if (g >= off) incl += v;
  }
  const int64_t per_head = __shfl(incl, M - 1);
  int64_t hs = per_head > 0 ? capacity / per_head : H;
  hs = per_head >= cap ? 0 : (hs < H ? hs : H);
  if (g < M) plan->off[g] = hs * (incl - bytes);
  if (g == 0) plan->heads = (int32_t)hs;
}

// Groups by decreasing size and the prefix count of (head, tile) items.
__global__ __launch_bounds__(kWave) void bwd_schedule_kernel(const int32_t* __restrict__ cu, int M, int H, int tile,
                                                           AttnSchedule* __restrict__ sched) {
  __shared__ int order_s[kMaxGroups];
  const int g = threadIdx.x;
  const int n = g < M ? cu[g + 1] - cu[g] : -1;
  if (g < M) {
    int rank = 0;
    for (int o = 0; o < M; ++o) {
      const int no = cu[o + 1] - cu[o];
      rank += (no > n) || (no == n && o < g);
    }
    order_s[rank] = g;
  }
  __syncthreads();
  int items = 0;
  if (g < M) {
    const int og = order_s[g];
    sched->order[g] = og;
    items = (cu[og + 1] - cu[og] + tile - 1) / tile * H;
  }
  int incl = items;
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (g >= off) incl += v;
  }
  if (g < M) sched->prefix[g + 1] = incl;
  if (g == 0) sched->prefix[0] = 0;
}

int64_t grid_for(int64_t items) {
  const int64_t run = (int64_t)kNumXcd * kRun;
  return ceil_div(items, run) * run;
}

template <int D>
int launch_bwd(const uint16_t* Qp, const uint16_t* Kp, const uint16_t* Vp, const uint16_t* dAp, const float* lse,
               const float* delta, const int32_t* cu, const int32_t* perm, AttnSchedule* sk, AttnSchedule* sq, int M,
               int64_t N, int H, float scale, uint16_t* dQ, uint16_t* dK, uint16_t* dV, const DsPlan* plan,
               uint8_t* ds, hipStream_t st) {
  const int64_t rs = (int64_t)H * D;
  const int64_t gk = grid_for((ceil_div(N, kDkvBN) + M) * H);
  const int64_t gq = grid_for((ceil_div(N, kDqBM) + M) * H);
  if (gk > 0x7fffffff || gq > 0x7fffffff) return MOGA_ERR_SHAPE;
  if (plan != nullptr)
    dkdv_kernel<D, true><<<dim3((unsigned)gk), kDkvWaves * kWave, 0, st>>>(Qp, Kp, Vp, dAp, lse, delta, cu, perm, sk,
                                                                          M, N, rs, scale, dK, dV, plan, ds);
  else
    dkdv_kernel<D, false><<<dim3((unsigned)gk), kDkvWaves * kWave, 0, st>>>(Qp, Kp, Vp, dAp, lse, delta, cu, perm, sk,
                                                                           M, N, rs, scale, dK, dV, nullptr, nullptr);
  MOGA_LAUNCH_CHECK();
  // Both dQ kernels are launched when dS may be staged; the plan (written on
  // the device) gives each head's work items to exactly one of them.
  dq_kernel<D><<<dim3((unsigned)gq), kDqWaves * kWave, 0, st>>>(Qp, Kp, Vp, dAp, lse, delta, cu, perm, sq, M, N, rs,
                                                                 scale, dQ, plan);
  MOGA_LAUNCH_CHECK();
  if (plan != nullptr) {
    dq_ds_kernel<D><<<dim3((unsigned)gq), kDqWaves * kWave, 0, st>>>(Kp, ds, plan, cu, perm, sq, M, rs, scale, dQ);
    MOGA_LAUNCH_CHECK();
  }
  return MOGA_OK;
}

}  // namespace
}  // namespace moga

extern "C" int moga_group_attention_backward(const void* Qp, const void* Kp, const void* Vp, const void* dOp,
                                             const float* lse, const float* delta, const int32_t* cu_seqlens,
                                             const int32_t* perm, int64_t N, int32_t H, int32_t D, int32_t M,
                                             float softmax_scale, void* dQ, void* dK, void* dV, void* ws,
                                             size_t ws_bytes, void* stream) {
  using namespace moga;
  if (!Qp || !Kp || !Vp || !dOp || !lse || !delta || !cu_seqlens || !perm || !dQ || !dK || !dV) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1 || H < 1 || D < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups || !valid_head_dims(H, D)) return MOGA_ERR_UNSUPPORTED;
  const size_t need = moga_workspace_bytes(MOGA_OP_ATTENTION_BACKWARD, N, M, H, D);
  if (!ws || ws_bytes < need) return MOGA_ERR_WORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  hipStream_t st = as_stream(stream);
  auto* sk = static_cast<AttnSchedule*>(ws);
  auto* sq = reinterpret_cast<AttnSchedule*>(static_cast<char*>(ws) + 1024);
  bwd_schedule_kernel<<<1, kWave, 0, st>>>(cu_seqlens, M, H, kDkvBN, sk);
  MOGA_LAUNCH_CHECK();
  bwd_schedule_kernel<<<1, kWave, 0, st>>>(cu_seqlens, M, H, kDqBM, sq);
  MOGA_LAUNCH_CHECK();
  // A workspace beyond the schedules may hold the staged dS; whether this
  // call's groups fit is decided on the device.
  DsPlan* plan = nullptr;
  uint8_t* ds = nullptr;
  if (ws_bytes > kDsDataOffset) {
    plan = reinterpret_cast<DsPlan*>(static_cast<char*>(ws) + kDsPlanOffset);
    ds = static_cast<uint8_t*>(ws) + kDsDataOffset;
    ds_plan_kernel<<<1, kWave, 0, st>>>(cu_seqlens, M, H, (int64_t)(ws_bytes - kDsDataOffset), plan);
    MOGA_LAUNCH_CHECK();
  }
  auto c = [](const void* p) { return static_cast<const uint16_t*>(p); };
  auto m = [](void* p) { return static_cast<uint16_t*>(p); };
  if (D == 128)
    return launch_bwd<128>(c(Qp), c(Kp), c(Vp), c(dOp), lse, delta, cu_seqlens, perm, sk, sq, M, N, H, scale, m(dQ),
                           m(dK), m(dV), plan, ds, st);
  return launch_bwd<64>(c(Qp), c(Kp), c(Vp), c(dOp), lse, delta, cu_seqlens, perm, sk, sq, M, N, H, scale, m(dQ),
                        m(dK), m(dV), plan, ds, st);
}

extern "C" size_t moga_attention_backward_staged_bytes(const int32_t* cu_seqlens_host, int32_t M, int32_t H) {
  using namespace moga;
  if (!cu_seqlens_host || M < 1 || M > kMaxGroups || H < 1) return 0;
  size_t total = kDsDataOffset;
  for (int g = 0; g < M; ++g) {
    const int64_t n = (int64_t)cu_seqlens_host[g + 1] - cu_seqlens_host[g];
    if (n < 0) return 0;
    const int64_t nb = (n + 31) >> 5, nbp = (nb + 1) & ~int64_t(1);
    if (nb > (int64_t(1) << 19)) return 0;
    total += (size_t)H * (size_t)nb * (size_t)nbp * kDsBlock;
  }
  return total;
}
