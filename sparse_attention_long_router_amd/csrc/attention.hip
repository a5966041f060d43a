// Group attention for gfx950: exact softmax attention inside every group, for
// the learned MoGA groups (variable length, permuted rows) and for the static
// STGA windows (fixed size, rows gathered by an index map).
// Page "MoGA: Mixture-of-Groups Attention for End-to-End Long Video
// Generation": Eq. 1 (softmax(q K^T / sqrt(d)) V) restricted to a group, as in
// the MoGA output equation ("Grouped Attention") and Algorithm 1 step 3; the
// static windows are those of the "Spatial-Temporal Group Attention (STGA)"
// section.  The online (running max / running sum) softmax is the one of the
// FlashAttention papers the pages cite; the tiling here is our own for CDNA4.
//
// Work item = (group, head, tile of 256 queries), one workgroup each.  A wave
// owns QB blocks of 32 queries (QB = 1: 8 waves, two per SIMD, so the
// hardware interleaves one wave's softmax with the other's MFMAs; QB = 2:
// 4 waves, one per SIMD, each K/V operand read feeding two MFMAs).  The static
// STGA windows use items of 128 queries instead (4 waves, two workgroups per
// CU): their items are short (2,340 keys in the long-video setting), and the
// second workgroup keeps the matrix cores busy through one item's table build,
// Q loads and output stores.  Per 64-key tile:
//   K and V rows arrive in LDS by 16-byte direct-to-LDS loads, XOR-swizzled
//   at 16-byte granularity (conflict-free reads), into four buffers with one
//   barrier per two tiles (the next pair streams in while this one computes;
//   the 128-query items, two workgroups to a CU's LDS, keep two buffers and
//   one barrier per tile); a tile's loads are issued after the first K
//   operand reads of the tile before it;
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the
//   wave's Q fragment held in registers) -- the C layout gives every lane one
//   query and 16 keys, so softmax statistics stay in-lane (the two wave
//   halves share a query and exchange one value with v_permlane32_swap);
//   softmax in float32 with exp2: the Q fragments carry the softmax scale in
//   log2 units, and the exponent offset is fixed before the key loop (none
//   at all when every row's first 32 scores are moderate, else their max),
//   so there is no accumulator rescaling; a work item whose denominator or
//   accumulator leaves the safe range is recomputed exactly;
//   O^T += V^T P^T with the same MFMA: B = P^T comes straight from the S^T
//   registers (the k-slot order of an MFMA is free as long as both operands
//   agree), A = V^T comes from row-major V in LDS through two
//   ds_read_b64_tr_b16 per operand, or, with V stored transposed per head
//   (MogaVtRows), from V^T tiles through one ds_read_b128.
// Items are handed out largest group first (longest-processing-time order) and
// dealt to the 8 XCDs in runs of 32 consecutive query tiles of one (group,
// head), so the tiles that stream the same K/V run side by side under one L2.
#include <type_traits>

#ifndef MOGA_ATTN_QB
#define MOGA_ATTN_QB 1
#endif
#include "moga_internal.h"

// LLVM's raw buffer load to LDS (buffer_load_dwordx4 ... lds): descriptor,
// LDS base (M0), bytes per lane, per-lane byte offset, scalar offset,
// immediate offset, cache policy.
typedef int32_t i32x4v __attribute__((ext_vector_type(4)));
__device__ void raw_buffer_load_lds(i32x4v rsrc, __attribute__((address_space(3))) void* lds, int size, int voffset,
                                    int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

namespace moga {
namespace {

constexpr int kBM = 256;  // queries per work item of the learned groups
constexpr int kQB = MOGA_ATTN_QB;                   // 32-query blocks per wave (1 or 2)
// Waves per workgroup: Rows::kQueries queries per work item, 32 * QB per wave.
template <class Rows, int QB>
constexpr int waves_for() { return Rows::kQueries / (32 * QB); }
constexpr int kBN = 64;                             // keys per LDS tile
// Consecutive items per XCD: 32, one per CU of the XCD, so a whole XCD
// streams one (group, head)'s K/V together through its L2.  At 190k tokens
// this reads 6.0 GB from HBM per launch against 10.5 GB with runs of 8, in
// the same time.
constexpr int kXcdRun = 32;
// Mean group size (tokens) below which the default forward path takes
// 128-query items (MogaVtQRows128).
constexpr int kShortGroup = 8192;
// LDS of one CU (gfx950), and the bytes __syncthreads_or reserves for its reduction.
constexpr int kCuLds = 160 * 1024;
constexpr int kSyncOrLds = 256;
// Key-row table entries of an index-map window (Rows::kTabKeys), sized so
// that the table and two K/V buffers (64 KB) fit in half of a CU's 160 KB of
// LDS and two workgroups share a CU: 4,096 (16 KB) for the shot-aware
// windows, which reach (win_t + 2 augment) frames of a tile; 3,840 for the
// static windows (2,340 keys in the long-video setting; the full 4,096 with
// the reduction below measured 2.5% slower there).  Larger windows evaluate the
// map per load.
template <class Rows>
constexpr int tab_keys() {
  if constexpr (Rows::kTable)
    return Rows::kTabKeys;
  else
    return 1;
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct Work {
  int len;      // keys of the group
  int nq;       // queries of the group (= len except for shot-aware windows)
  int q0;       // first query (group-local) of this item
  int head;
  int64_t row0; // MoGA: first permuted row of the group
  int t0, y0, x0;  // STGA: window origin
  int nt, npre, pre_off, nxt_off;  // shot-aware STGA: window frames, frames before, frame offsets
};

// Learned groups: rows of group g are cu[g] .. cu[g+1]-1 of the permuted tensors.
struct MogaRows {
  static constexpr int kQueries = kBM;
  static constexpr bool kIndirect = false;
  static constexpr bool kContiguous = true;  // key row i of a group is row0 + i
  static constexpr bool kTable = false;
  static constexpr bool kVt = false;
  const int32_t* cu;
  const AttnSchedule* sched;
  int M, H;
  // item -> (group, head, query tile of QT queries); the schedule counts
  // tiles of the same size
  template <int QT>
  __device__ __forceinline__ bool decode_tiles(int item, Work& w) const {
    const int total = sched->prefix[M];
    if (item >= total) return false;
    int i = 0;
    while (i + 1 < M && sched->prefix[i + 1] <= item) ++i;
    const int g = sched->order[i];
    const int local = item - sched->prefix[i];
    const int lo = cu[g];
    const int len = cu[g + 1] - lo;
    const int nt = (len + QT - 1) / QT;
    w.len = len;
    w.nq = len;
    w.head = local / nt;
    w.q0 = (local - w.head * nt) * QT;
    w.row0 = lo;
    return true;
  }
  __device__ __forceinline__ bool decode(int item, Work& w) const { return decode_tiles<kBM>(item, w); }
  __device__ __forceinline__ int64_t row(const Work& w, int i) const { return w.row0 + i; }
  __device__ __forceinline__ int64_t key(const Work& w, int i) const { return w.row0 + i; }
};

// Learned groups with V stored transposed per head: Vt [H][D][ldv], the keys
// of one channel contiguous and zero-padded (moga_permute_vt writes it).  A V operand of the
// P V product is then one 16-byte LDS read instead of two transposing reads.
struct MogaVtRows {
  static constexpr int kQueries = kBM;
  static constexpr bool kIndirect = false;
  [[maybe_unused]] static constexpr bool kContiguous = true;  // as MogaRows; the kVt path takes precedence
  static constexpr bool kTable = false;
  static constexpr bool kVt = true;
  MogaRows base;
  int64_t ldv;  // tokens per V^T row (N plus zero padding)
  __device__ __forceinline__ bool decode(int item, Work& w) const { return base.decode(item, w); }
  __device__ __forceinline__ int64_t row(const Work& w, int i) const { return w.row0 + i; }
  __device__ __forceinline__ int64_t key(const Work& w, int i) const { return w.row0 + i; }
};

// MogaVtRows with the queries read in original token order: query i of a
// group is token perm[row0 + i] of the unpermuted Q, so only K and V^T are
// gathered.  The output row is that same token (kEpiGatedInPlace).
struct MogaVtQRows : MogaVtRows {
  const int32_t* perm;
  __device__ __forceinline__ int64_t row(const Work& w, int i) const { return perm[w.row0 + i]; }
};

// MogaVtQRows in 128-query items (four waves, two workgroups per CU, as the
// STGA windows): for short groups, where each item's fixed work (first
// tiles, query rows, epilogue) weighs more and one item's fixed work then
// runs beside the other's tiles.  Long groups keep 256-query items, which
// stream every K/V tile for twice as many queries.
struct MogaVtQRows128 : MogaVtQRows {
  static constexpr int kQueries = 128;
  __device__ __forceinline__ bool decode(int item, Work& w) const { return base.decode_tiles<128>(item, w); }
};

// Learned groups read in place (gather on load): permuted row j of a group is
// original token perm[j], so Q, K and V are the unpermuted tensors and no
// gathered copies exist.  Key rows are fetched a tile ahead (kIndirect).
struct MogaPermRows {
  static constexpr int kQueries = kBM;
  static constexpr bool kIndirect = true;
  static constexpr bool kContiguous = false;
  static constexpr bool kTable = false;
  static constexpr bool kVt = false;
  MogaRows base;
  const int32_t* perm;
  __device__ __forceinline__ bool decode(int item, Work& w) const { return base.decode(item, w); }
  __device__ __forceinline__ int64_t row(const Work& w, int i) const { return perm[w.row0 + i]; }
  __device__ __forceinline__ int32_t key_index(const Work& w, int i) const { return perm[w.row0 + i]; }
};

// i / d and i % d for 0 <= i < 2^24 and 0 < d < 2^24 from a float reciprocal
// of d (rounded once): the float quotient is within 1 of the exact one and a
// single correction step fixes it.  Cheaper than the integer division
// sequence in the per-item key tables of the index-map windows.
__device__ __forceinline__ int fast_divmod(int i, int d, float inv_d, int& rem) {
  int q = (int)((float)i * inv_d);
  int r = i - q * d;
  if (r < 0) {
    --q;
    r += d;
  } else if (r >= d) {
    ++q;
    r -= d;
  }
  rem = r;
  return q;
}

// Static windows over frame-major tokens n = (t*Hs + y)*Ws + x.
struct StgaRows {
  // 128-query items (four waves): two workgroups share a CU, so one item's
  // table, Q loads and output stores overlap the other's tiles.
  static constexpr int kQueries = 128;
  static constexpr int kTabKeys = 3840;
  static constexpr bool kIndirect = false;
  static constexpr bool kContiguous = false;
  static constexpr bool kTable = true;  // key rows tabulated in LDS once per item
  static constexpr bool kVt = false;
  int Hs, Ws, win_t, tile_h, tile_w, nty, ntx, tiles_per_group, H, items;
  uint32_t tab_bytes;  // byte size of one K/V tensor when below 2^31 (key table of byte offsets), else 0
  float inv_area, inv_tw;  // 1 / (tile_h * tile_w), 1 / tile_w
  __device__ __forceinline__ bool decode(int item, Work& w) const {
    if (item >= items) return false;
    const int per_group = H * tiles_per_group;
    const int grp = item / per_group;
    const int rem = item - grp * per_group;
    w.head = rem / tiles_per_group;
    w.q0 = (rem - w.head * tiles_per_group) * kQueries;
    w.len = win_t * tile_h * tile_w;
    w.nq = w.len;
    const int tw = grp / (nty * ntx);
    const int r2 = grp - tw * (nty * ntx);
    const int ty = r2 / ntx;
    w.t0 = tw * win_t;
    w.y0 = ty * tile_h;
    w.x0 = (r2 - ty * ntx) * tile_w;
    w.row0 = 0;
    return true;
  }
  __device__ __forceinline__ int64_t row(const Work& w, int i) const {
    int rem, xx;
    const int tt = fast_divmod(i, tile_h * tile_w, inv_area, rem);
    const int yy = fast_divmod(rem, tile_w, inv_tw, xx);
    return ((int64_t)(w.t0 + tt) * Hs + (w.y0 + yy)) * Ws + (w.x0 + xx);
  }
  __device__ __forceinline__ int64_t key(const Work& w, int i) const { return row(w, i); }
};

// One temporal window of the shot-aware STGA: frames t0 .. t0+nt-1 of one
// shot, plus frames pre0 .. pre0+npre-1 of the previous shot and
// nxt0 .. nxt0+nnxt-1 of the next one, whose tokens join the keys and values
// only.
struct ShotWindow {
  int t0, nt, pre0, npre, nxt0, nnxt;
};

// Shot-aware windows: queries are the window's own frames inside one spatial
// tile; keys are those tokens followed by the same tile of the extra frames.
// Items: window-major, then spatial tile, head and query tile, so the query
// tiles sharing one key set are consecutive (and land on one XCD).
struct ShotRows {
  static constexpr int kQueries = 128;  // as StgaRows: two workgroups per CU
  static constexpr int kTabKeys = 4096;
  static constexpr bool kIndirect = false;
  static constexpr bool kContiguous = false;
  static constexpr bool kTable = true;
  static constexpr bool kVt = false;
  const ShotWindow* win;
  const int* nwin;
  int Hs, Ws, tile_h, tile_w, ntx, nspatial, tpg, H;
  uint32_t tab_bytes;  // as in StgaRows
  float inv_area, inv_tw;  // as in StgaRows
  __device__ __forceinline__ bool decode(int item, Work& w) const {
    const int per_win = nspatial * H * tpg;
    const int wi = item / per_win;
    if (wi >= *nwin) return false;
    int rem = item - wi * per_win;
    const int sp = rem / (H * tpg);
    rem -= sp * (H * tpg);
    w.head = rem / tpg;
    w.q0 = (rem - w.head * tpg) * kQueries;
    const ShotWindow sw = win[wi];
    const int area = tile_h * tile_w;
    w.nq = sw.nt * area;
    if (w.q0 >= w.nq) return false;
    // key frame tt: t0 + tt inside the window, then pre0 + (tt - nt), then nxt0 + (tt - nt - npre)
    w.nt = sw.nt;
    w.npre = sw.nt + sw.npre;
    w.pre_off = sw.pre0 - sw.nt;
    w.nxt_off = sw.nxt0 - w.npre;
    w.len = (sw.nt + sw.npre + sw.nnxt) * area;
    w.t0 = sw.t0;
    const int ty = sp / ntx;
    w.y0 = ty * tile_h;
    w.x0 = (sp - ty * ntx) * tile_w;
    w.row0 = 0;
    return true;
  }
  __device__ __forceinline__ int64_t at(const Work& w, int frame, int i) const {
    int xx;
    const int yy = fast_divmod(i, tile_w, inv_tw, xx);
    return ((int64_t)frame * Hs + (w.y0 + yy)) * Ws + (w.x0 + xx);
  }
  __device__ __forceinline__ int64_t row(const Work& w, int i) const {
    int rem;
    const int tt = fast_divmod(i, tile_h * tile_w, inv_area, rem);
    return at(w, w.t0 + tt, rem);
  }
  __device__ __forceinline__ int64_t key(const Work& w, int i) const {
    int rem;
    const int tt = fast_divmod(i, tile_h * tile_w, inv_area, rem);
    const int t0 = w.t0, pre_off = w.pre_off, nxt_off = w.nxt_off;  // values, not a select of field addresses
    const int off = tt < w.npre ? pre_off : nxt_off;
    const int frame = tt + (tt < w.nt ? t0 : off);
    return at(w, frame, rem);
  }
};

// 16-byte chunk swizzles of the K and V tiles in LDS (cpr = chunks per row).
__device__ __forceinline__ int kswz(int r, int cpr) { return r & (cpr - 1); }
__device__ __forceinline__ int vswz(int r, int cpr) { return ((r & 3) << 2) & (cpr - 1); }

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

// Softmax bookkeeping of one 32-query block (one query per lane; the two wave
// halves hold the same query).  The exponent offset m_ref is fixed from the
// row's first 32 keys before the key loop and never moves, so the output
// accumulator is never rescaled and no per-tile row max is needed.  Weights
// above 1 (later scores above the first keys' max) keep their relative
// precision in float32 and bf16; only a denominator that reaches kLimit
// (2^64) or overflows could lose the output, and the work item is then
// recomputed with the exact row max (see attn_kernel).
struct RowState {
  float m_ref;  // exponent offset (log2 domain)
  float l;      // this lane's share of the denominator
};
constexpr float kLimit = 18446744073709551616.0f;  // 2^64
constexpr float kTiny = 5.42101086242752217e-20f;     // 2^-64
constexpr float kFastLo = -64.f, kFastHi = 32.f;     // offset-free range of the first scores (log2 units)

// max / sum of a value over the two wave halves (lanes c and c+32 share a query)
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Issue one K/V tile (kBN rows starting at group-local key k0) into LDS with
// 16-byte direct-to-LDS loads.  Lane i of a load lands at LDS base + 16*i, so
// the swizzle is applied on the source side: the lane writing physical chunk p
// of row r fetches logical chunk p ^ swz(r).  Rows past the group end repeat
// the last row (finite data; their scores are masked).
template <int D, int NW, class Rows>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                           uint16_t* Ks, uint16_t* Vs, const Rows& rows, const Work& w,
                                           int64_t row_stride, int64_t hoff, int k0, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int LOADS = kBN * CPR / (NW * kWave);  // per wave, per tensor
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int q = (wave * LOADS + j) * kWave + lane;  // chunk index inside the tile
    const int r = q / CPR, p = q % CPR;
    int key = k0 + r;
    key = key < w.len ? key : w.len - 1;
    const int64_t base = rows.key(w, key) * row_stride + hoff;
    const int lds_off = (wave * LOADS + j) * kWave * 8;  // uint16 elements, wave-uniform
    __builtin_amdgcn_global_load_lds((global_void*)(K + base + (p ^ kswz(r, CPR)) * 8), (lds_void*)(Ks + lds_off),
                                     16, 0, 0);
    __builtin_amdgcn_global_load_lds((global_void*)(V + base + (p ^ vswz(r, CPR)) * 8), (lds_void*)(Vs + lds_off),
                                     16, 0, 0);
  }
}

// Table variant of issue_tile for index-map windows: the token row of every
// key was written to LDS (tab) once per work item, so the per-tile issue reads
// it instead of evaluating the (t, y, x) map per 16-byte chunk.
template <int D, int NW>
__device__ __forceinline__ void issue_tile_tab(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                               uint16_t* Ks, uint16_t* Vs, const int32_t* tab, int len,
                                               int64_t row_stride, int64_t hoff, int k0, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int LOADS = kBN * CPR / (NW * kWave);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int q = (wave * LOADS + j) * kWave + lane;
    const int r = q / CPR, p = q % CPR;
    int key = k0 + r;
    key = key < len ? key : len - 1;
    const int64_t base = (int64_t)tab[key] * row_stride + hoff;
    const int lds_off = (wave * LOADS + j) * kWave * 8;
    __builtin_amdgcn_global_load_lds((global_void*)(K + base + (p ^ kswz(r, CPR)) * 8), (lds_void*)(Ks + lds_off),
                                     16, 0, 0);
    __builtin_amdgcn_global_load_lds((global_void*)(V + base + (p ^ vswz(r, CPR)) * 8), (lds_void*)(Vs + lds_off),
                                     16, 0, 0);
  }
}

// Byte-offset table variant: tab holds each key's row offset in bytes (padded
// to whole tiles), the tensors are covered by one buffer descriptor each and
// the head offset rides in the scalar offset.
template <int D, int NW>
__device__ __forceinline__ void issue_tile_tab32(i32x4v krs, i32x4v vrs, uint16_t* Ks, uint16_t* Vs,
                                                 const int32_t* tab, int soff, int k0, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int LOADS = kBN * CPR / (NW * kWave);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int q = (wave * LOADS + j) * kWave + lane;
    const int r = q / CPR, p = q % CPR;
    const int off = tab[k0 + r];
    const int lds_off = (wave * LOADS + j) * kWave * 8;
    raw_buffer_load_lds(krs, (lds_void*)(Ks + lds_off), 16, off + ((p ^ kswz(r, CPR)) << 4), soff, 0, 0);
    raw_buffer_load_lds(vrs, (lds_void*)(Vs + lds_off), 16, off + ((p ^ vswz(r, CPR)) << 4), soff, 0, 0);
  }
}

// Contiguous-row variant of issue_tile: buffer loads straight to LDS.  The
// tile's first row and the group's remaining bytes live in a scalar buffer
// descriptor, so a lane's byte offset (row in tile, swizzled chunk) is the
// same for every tile and no per-tile address arithmetic runs on the VALU;
// rows past the group end fail the descriptor's range check and land in LDS
// as zeros (their scores are masked).
// Descriptor of rows [first, first + n) of one head: base address, stride 0,
// byte range, and the gfx9 raw-buffer data format word.
__device__ __forceinline__ i32x4v row_range_rsrc(const uint16_t* base, int64_t n_rows, int64_t row_bytes,
                                                 int bytes_per_row) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  int64_t range = n_rows > 0 ? (n_rows - 1) * row_bytes + bytes_per_row : 0;
  range = range < 0xffffffffll ? range : 0xffffffffll;
  i32x4v r;
  r[0] = (int32_t)(uint32_t)a;
  r[1] = (int32_t)(uint32_t)(a >> 32);
  r[2] = (int32_t)(uint32_t)range;
  r[3] = 0x00020000;
  return r;
}

template <int D, int NW>
__device__ __forceinline__ void issue_tile_buf(i32x4v krs, i32x4v vrs, uint16_t* Ks, uint16_t* Vs,
                                               int64_t row_stride, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int LOADS = kBN * CPR / (NW * kWave);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int q = (wave * LOADS + j) * kWave + lane;
    const int r = q / CPR, p = q % CPR;
    const int rb = r * (int)row_stride * 2;
    const int lds_off = (wave * LOADS + j) * kWave * 8;
    raw_buffer_load_lds(krs, (lds_void*)(Ks + lds_off), 16, rb + ((p ^ kswz(r, CPR)) << 4), 0, 0, 0);
    raw_buffer_load_lds(vrs, (lds_void*)(Vs + lds_off), 16, rb + ((p ^ vswz(r, CPR)) << 4), 0, 0, 0);
  }
}

// Transposed-V tiles (MogaVtRows).  The K rows of each 16-key block sit in
// LDS with key bits 2 and 3 swapped (physical row r holds key swap23(r)): the
// score rows one lane half holds for a 16-key MFMA step are then 8
// consecutive keys, which is exactly what one 16-byte read of a V^T row
// supplies.  The V^T tile is D channel rows of the tile's 64 keys (128
// bytes); chunk p of channel row r sits at chunk p ^ ((r >> 1) & 7), which
// keeps any 16 consecutive rows conflict-free for the 16-byte reads.
__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
__device__ __forceinline__ int vtswz(int r) { return (r >> 1) & 7; }

template <int D, int NW>
__device__ __forceinline__ void issue_tile_vt(i32x4v krs, i32x4v vrs, uint16_t* Ks, uint16_t* Vs,
                                              int64_t row_stride, int64_t ldv, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int LOADS = kBN * CPR / (NW * kWave);  // the V^T tile (D rows x 8 chunks) has as many chunks
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int q = (wave * LOADS + j) * kWave + lane;
    const int lds_off = (wave * LOADS + j) * kWave * 8;
    const int r = q / CPR, p = q % CPR;  // K: physical row r, chunk p
    raw_buffer_load_lds(krs, (lds_void*)(Ks + lds_off), 16,
                        swap23(r) * (int)row_stride * 2 + ((p ^ kswz(r, CPR)) << 4), 0, 0, 0);
    const int vr = q >> 3, vp = q & 7;  // V^T: channel row vr, chunk vp
    raw_buffer_load_lds(vrs, (lds_void*)(Vs + lds_off), 16, vr * (int)ldv * 2 + ((vp ^ vtswz(vr)) << 4), 0, 0, 0);
  }
}

// Gather-on-load variant of issue_tile: the token row of every chunk this
// lane loads was fetched beforehand (fetch_keys) into kidx.
template <int D, int NW>
constexpr int tile_loads() { return kBN * (D / 8) / (NW * kWave); }

template <int D, int NW, class Rows>
__device__ __forceinline__ void fetch_keys(const Rows& rows, const Work& w, int k0, int wave, int lane,
                                           int32_t (&kidx)[tile_loads<D, NW>()]) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int j = 0; j < tile_loads<D, NW>(); ++j) {
    const int r = ((wave * tile_loads<D, NW>() + j) * kWave + lane) / CPR;
    int key = k0 + r;
    key = key < w.len ? key : w.len - 1;
    kidx[j] = rows.key_index(w, key);
  }
}

template <int D, int NW>
__device__ __forceinline__ void issue_tile_idx(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                               uint16_t* Ks, uint16_t* Vs, const int32_t (&kidx)[tile_loads<D, NW>()],
                                               int64_t row_stride, int64_t hoff, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int LOADS = tile_loads<D, NW>();
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int q = (wave * LOADS + j) * kWave + lane;
    const int r = q / CPR, p = q % CPR;
    const int64_t base = (int64_t)kidx[j] * row_stride + hoff;
    const int lds_off = (wave * LOADS + j) * kWave * 8;
    __builtin_amdgcn_global_load_lds((global_void*)(K + base + (p ^ kswz(r, CPR)) * 8), (lds_void*)(Ks + lds_off),
                                     16, 0, 0);
    __builtin_amdgcn_global_load_lds((global_void*)(V + base + (p ^ vswz(r, CPR)) * 8), (lds_void*)(Vs + lds_off),
                                     16, 0, 0);
  }
}

// How a score becomes an exponent: kExpFree: s' (the Q fragments carry the
// softmax scale in log2 units, no offset); kExpSub: s' - m_ref (scaled Q,
// offset); kExpFma: s * scale_log2 - m_ref (unscaled Q: the training forward).
enum { kExpFree = 0, kExpSub = 1, kExpFma = 2 };

// Softmax step of one query block over one 32-key half of a tile: bf16 P^T
// operands of the half's two 16-key MFMA steps go to pb, their sum to st.l.
// s: reg r is key 8*(r/4) + 4*hh + r%4 of the half (masked keys are -inf).
template <int kExp>
__device__ __forceinline__ void softmax_half(const f32x16& s, RowState& st, float scale_log2, bf16x8 (&pb)[2]) {
  float rs = st.l;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = s[8 * t + j];
      if constexpr (kExp == kExpSub) x -= st.m_ref;
      if constexpr (kExp == kExpFma) x = fmaf(x, scale_log2, -st.m_ref);
      const float p = __builtin_amdgcn_exp2f(x);
      pb[t][j] = (__bf16)p;
      rs += p;
    }
  st.l = rs;
}

// S^T of one 32-key half kb for the wave's QB query blocks; each K operand
// read from LDS feeds QB MFMAs.  Reg r of s[b] is key kb*32 + 8*(r/4) + 4*hh + r%4.
struct NoOp {
  __device__ __forceinline__ void operator()() const {}
};
template <int D, int QB, class AfterLoads = NoOp>
__device__ __forceinline__ void qk_half(const uint16_t* Ks, const bf16x8 (&qf)[QB][D / 16], int kb, int lane,
                                        f32x16 (&s)[QB], AfterLoads after_loads = {}) {
  constexpr int CPR = D / 8;
  const int hh = lane >> 5, krow = kb * 32 + (lane & 31);
#pragma unroll
  for (int b = 0; b < QB; ++b) s[b] = f32x16{};

  // All K operands of the half first, then the dependent MFMA chain: without
  // the fence the scheduler reuses one operand register and exposes an LDS
  // round trip before every MFMA of the chain.
  bf16x8 ka[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    ka[st] = *reinterpret_cast<const bf16x8*>(Ks + krow * D + ((2 * st + hh) ^ kswz(krow, CPR)) * 8);
  after_loads();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
#pragma unroll
    for (int b = 0; b < QB; ++b) s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st], qf[b][st], s[b], 0, 0, 0);
  }
}

// O^T += V^T P^T for one 32-key half kb and the wave's query blocks; each V^T
// operand (two transposing LDS reads) feeds QB MFMAs.  kOneOffset forms each
// read address as the buffer plus one offset: with the V buffers in their own
// arrays this keeps the reads traceable to their buffer, so the compiler does
// not wait for the loads in flight into the other buffer.
template <int D, int QB, bool kOneOffset = false>
__device__ __forceinline__ void pv_half(const uint16_t* Vs, const bf16x8 (&p)[QB][2], int kb, int lane,
                                        f32x16 (&o)[QB][D / 32]) {
  constexpr int CPR = D / 8;
  const int hh = lane >> 5;
  const int tr_r = (lane & 15) >> 2, tr_q = lane & 3, tr_g = (lane >> 4) & 1;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r1 = kb * 32 + 16 * t + 4 * hh + tr_r;
    const int r2 = r1 + 8;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = 32 * db + 16 * tr_g + 4 * tr_q;
      const int ch = col >> 3, within = col & 7;
      const uint16_t* a1 = kOneOffset ? Vs + (r1 * D + ((ch ^ vswz(r1, CPR)) << 3) + within)
                                      : Vs + r1 * D + ((ch ^ vswz(r1, CPR)) << 3) + within;
      const uint16_t* a2 = kOneOffset ? Vs + (r2 * D + ((ch ^ vswz(r2, CPR)) << 3) + within)
                                      : Vs + r2 * D + ((ch ^ vswz(r2, CPR)) << 3) + within;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a1);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a2);
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int b = 0; b < QB; ++b) o[b][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[b][t], o[b][db], 0, 0, 0);
    }
  }
}

// pv_half with V^T in LDS (MogaVtRows): the operand of channel block db and
// 16-key step t is one 16-byte read of channel row 32*db + lane%32, keys
// 32*kb + 16*t + 8*hh .. +7, matching P's slots under the swapped K rows.
template <int D, int QB>
__device__ __forceinline__ void pv_half_t(const uint16_t* Vs, const bf16x8 (&p)[QB][2], int kb, int lane,
                                          f32x16 (&o)[QB][D / 32]) {
  const int hh = lane >> 5;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int r = 32 * db + (lane & 31);
      const int c = (4 * kb + 2 * t + hh) ^ vtswz(r);
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vs + r * kBN + c * 8);
#pragma unroll
      for (int b = 0; b < QB; ++b) o[b][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[b][t], o[b][db], 0, 0, 0);
    }
  }
}

template <bool kMask, int QB, bool kPermK = false>
__device__ __forceinline__ void mask_half(f32x16 (&s)[QB], int key0, int len, int hh) {
  if constexpr (kMask) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int m = 8 * (r >> 2) + 4 * hh + (r & 3);  // LDS row of reg r in the half
      if constexpr (kPermK) m = swap23(m);      // its key
      if (key0 + m >= len) {
#pragma unroll
        for (int b = 0; b < QB; ++b) s[b][r] = -INFINITY;
      }
    }
  }
}

// One 64-key tile for the wave's query blocks, in 32-key halves:
//   QK(h0) QK(h1) | softmax(h0) PV(h0) | softmax(h1) PV(h1)
template <int D, int QB, bool kMask, bool kVt, int kExp, bool kOneOffset = false, class AfterLoads = NoOp>
__device__ __forceinline__ void tile_step(const uint16_t* Ks, const uint16_t* Vs, int k0, int len,
                                          const bf16x8 (&qf)[QB][D / 16], f32x16 (&o)[QB][D / 32],
                                          RowState (&rs)[QB], float scale_log2, int lane,
                                          AfterLoads after_loads = {}) {
  const int hh = lane >> 5;
  f32x16 s0[QB], s1[QB];
  bf16x8 p[QB][2];
  __builtin_amdgcn_s_setprio(1);
  // The score chains issue at raised wave priority: when both waves of a SIMD
  // have an instruction ready, the one with MFMAs to issue goes first.
  qk_half<D, QB>(Ks, qf, 0, lane, s0, after_loads);
  qk_half<D, QB>(Ks, qf, 1, lane, s1);
  __builtin_amdgcn_s_setprio(0);
  mask_half<kMask, QB, kVt>(s0, k0, len, hh);
#pragma unroll
  for (int b = 0; b < QB; ++b) softmax_half<kExp>(s0[b], rs[b], scale_log2, p[b]);
  if constexpr (kVt)
    pv_half_t<D, QB>(Vs, p, 0, lane, o);
  else
    pv_half<D, QB, kOneOffset>(Vs, p, 0, lane, o);
  mask_half<kMask, QB, kVt>(s1, k0 + 32, len, hh);
#pragma unroll
  for (int b = 0; b < QB; ++b) softmax_half<kExp>(s1[b], rs[b], scale_log2, p[b]);
  if constexpr (kVt)
    pv_half_t<D, QB>(Vs, p, 1, lane, o);
  else
    pv_half<D, QB, kOneOffset>(Vs, p, 1, lane, o);
}

// Row maxima and sums (the first pass of the exact recomputation): per lane
// half, the running max mx and the sum l of 2^(s' - mx), rescaled when the
// max grows.  sc converts an MFMA score to log2 units.
template <int D, int QB, bool kMask, bool kVt>
__device__ __forceinline__ void tile_stats(const uint16_t* Ks, int k0, int len, const bf16x8 (&qf)[QB][D / 16],
                                           float sc, float (&mx)[QB], float (&l)[QB], int lane) {
  const int hh = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 s[QB];
    qk_half<D, QB>(Ks, qf, kb, lane, s);
    mask_half<kMask, QB, kVt>(s, k0 + 32 * kb, len, hh);
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      float m = mx[b];
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, s[b][r] * sc);
      const float ms = m == -INFINITY ? 0.f : m;  // a lane half with every key so far masked
      float add = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) add += __builtin_amdgcn_exp2f(s[b][r] * sc - ms);
      l[b] = l[b] * __builtin_amdgcn_exp2f(mx[b] - ms) + add;
      mx[b] = m;
    }
  }
}

// Output stage of the attention kernel:
//   kEpiPlain:  O[row] = attn                                  (permuted order)
//   kEpiScaled: O[row] = alpha * attn + beta * O[row]          (STGA)
//   kEpiGated:  n = perm[row]; O[n] = gate[n] * attn + beta * O[n]
//               (the gated unpermute fused into the attention)
//   kEpiGatedInPlace: the row already is the original token n (gather on
//               load); O[n] = gate[n] * attn + beta * O[n]
//   kEpiPlainLse: as kEpiPlain, and lse[head][row] = log sum_j exp(scale s_j)
//               (natural log) for the backward pass
enum { kEpiPlain = 0, kEpiScaled = 1, kEpiGated = 2, kEpiGatedInPlace = 3, kEpiPlainLse = 4 };
struct Epilogue {
  float alpha, beta;
  const int32_t* perm;
  const float* gate;
  float* lse;        // kEpiPlainLse: [H][n_rows]
  int64_t n_rows;
};

template <int D, int QB, class Rows, int kEpi>
__global__ __launch_bounds__((waves_for<Rows, QB>() * kWave), 2) void attn_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, int64_t row_stride, float scale_log2, Epilogue epi, Rows rows) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int NW = waves_for<Rows, QB>();
  // The Q fragments carry the softmax scale in log2 units, except in the
  // training forward: its saved log-sum-exp is paired with the unscaled Q by
  // the backward pass.
  constexpr bool kPre = kEpi != kEpiPlainLse;
  // 256-query items: four K/V buffers in one array and one barrier per two
  // tiles, K buffers first, so that every K read (and every V read) is one
  // base address plus an offset below 64 KB.  128-query items (two
  // workgroups per CU): two buffers and one barrier per tile, the buffer
  // being read and the one being loaded in separate arrays -- the compiler
  // then sees that the transposing V reads do not depend on the loads in
  // flight (in one array it waits for all of them before such a read).
  constexpr bool kPair = Rows::kQueries == kBM;
  constexpr int NBUF = kPair ? 4 : 2;
  __shared__ __attribute__((aligned(1024))) uint16_t kv_lds[kPair ? 2 * NBUF : 2][kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t kv_lds1[kPair ? 1 : 2][kBN * D];
  uint16_t *Ks0, *Ks1, *Vs0, *Vs1;
  if constexpr (kPair) {
    Ks0 = kv_lds[0];
    Ks1 = kv_lds[1];
    Vs0 = kv_lds[NBUF];
    Vs1 = kv_lds[NBUF + 1];
  } else {  // buffer 0 = kv_lds (K, V), buffer 1 = kv_lds1 (K, V)
    Ks0 = kv_lds[0];
    Vs0 = kv_lds[1];
    Ks1 = kv_lds1[0];
    Vs1 = kv_lds1[1];
  }
  [[maybe_unused]] uint16_t* const Ks2 = kv_lds[kPair ? 2 : 0];
  [[maybe_unused]] uint16_t* const Ks3 = kv_lds[kPair ? 3 : 0];
  [[maybe_unused]] uint16_t* const Vs2 = kv_lds[kPair ? NBUF + 2 : 0];
  [[maybe_unused]] uint16_t* const Vs3 = kv_lds[kPair ? NBUF + 3 : 0];

  Work w;
  if (!rows.decode(xcd_remap(blockIdx.x, kXcdRun), w)) return;  // uniform per block

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: scalar address arithmetic
  const int hh = lane >> 5, c = lane & 31;
  const int64_t hoff = (int64_t)w.head * D;
  // The head's byte offset within a row, the scalar offset of the table
  // loads.  Made uniform explicitly: the item decode divides on the VALU, and a
  // value the compiler cannot prove uniform wraps every such load in a loop
  // over the distinct values.
  [[maybe_unused]] const int hoff_bytes = __builtin_amdgcn_readfirstlane((int)(hoff * 2));
  const int nfull = w.len / kBN;            // tiles without a group end inside
  const int ntiles = (w.len + kBN - 1) / kBN;

  // Index-map windows: tabulate every key's token row once (up to tab_keys<Rows>()).
  __shared__ int32_t ktab[tab_keys<Rows>()];
  [[maybe_unused]] const bool use_tab = Rows::kTable && w.len <= tab_keys<Rows>();  // uniform per block
  [[maybe_unused]] bool use_tab32 = false;
  if constexpr (Rows::kTable) use_tab32 = use_tab && rows.tab_bytes != 0;
  if constexpr (Rows::kTable) {
    if (use_tab) {
      if (use_tab32) {  // byte offsets of the rows, padded to whole tiles with the last row
        const int padded = (w.len + kBN - 1) / kBN * kBN;
        for (int i = tid; i < padded; i += NW * kWave)
          ktab[i] = (int32_t)(rows.key(w, i < w.len ? i : w.len - 1) * row_stride * 2);
      } else {
        for (int i = tid; i < w.len; i += NW * kWave) ktab[i] = (int32_t)rows.key(w, i);
      }
      __syncthreads();
    }
  }

  // Tile t's K/V loads; with gather on load, also fetch tile t+1's key rows.
  [[maybe_unused]] int32_t kidx[tile_loads<D, NW>()];
  auto issue = [&](uint16_t* Kd, uint16_t* Vd, int t) {
    if constexpr (Rows::kVt) {
      // V^T rows of this head: channel d is V + (head * D + d) * ldv.  The
      // tile's 64 keys lie inside the row (its padding is zeros), so the
      // descriptor covers whole tiles; keys past the group end are masked.
      const int64_t k0 = w.row0 + (int64_t)t * kBN;
      issue_tile_vt<D, NW>(row_range_rsrc(K + k0 * row_stride + hoff, w.len - t * kBN, row_stride * 2, D * 2),
                           row_range_rsrc(V + (int64_t)w.head * D * rows.ldv + k0, D, rows.ldv * 2, kBN * 2),
                           Kd, Vd, row_stride, rows.ldv, wave, lane);
    } else if constexpr (Rows::kContiguous) {
      const int64_t first = (w.row0 + (int64_t)t * kBN) * row_stride + hoff;
      const int64_t n_rows = w.len - t * kBN;
      issue_tile_buf<D, NW>(row_range_rsrc(K + first, n_rows, row_stride * 2, D * 2),
                            row_range_rsrc(V + first, n_rows, row_stride * 2, D * 2), Kd, Vd, row_stride, wave, lane);
    } else if constexpr (Rows::kIndirect) {
      issue_tile_idx<D, NW>(K, V, Kd, Vd, kidx, row_stride, hoff, wave, lane);
      if (t + 1 < ntiles) fetch_keys<D, NW>(rows, w, (t + 1) * kBN, wave, lane, kidx);
    } else if (use_tab) {
      if (use_tab32)
        issue_tile_tab32<D, NW>(row_range_rsrc(K, 1, 0, (int)rows.tab_bytes),
                                row_range_rsrc(V, 1, 0, (int)rows.tab_bytes), Kd, Vd, ktab, hoff_bytes,
                                t * kBN, wave, lane);
      else
        issue_tile_tab<D, NW>(K, V, Kd, Vd, ktab, w.len, row_stride, hoff, t * kBN, wave, lane);
    } else {
      issue_tile<D, NW>(K, V, Kd, Vd, rows, w, row_stride, hoff, t * kBN, wave, lane);
    }
  };
  auto issue_first = [&]() {
    if constexpr (Rows::kIndirect) fetch_keys<D, NW>(rows, w, 0, wave, lane, kidx);
    issue(Ks0, Vs0, 0);
    if constexpr (kPair) {
      if (1 < ntiles) issue(Ks1, Vs1, 1);
    }
  };
  issue_first();

  // this lane's two queries (blocks b = 0, 1) and their Q fragments
  int64_t qrow[QB];
  bool qvalid[QB];
  bf16x8 qf[QB][KSTEPS];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int qi = w.q0 + (wave * QB + b) * 32 + c;
    qvalid[b] = qi < w.nq;
    qrow[b] = rows.row(w, qvalid[b] ? qi : w.nq - 1);
    const uint16_t* qp = Q + qrow[b] * row_stride + hoff + 8 * hh;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      qf[b][s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
      if constexpr (kPre) {
#pragma unroll
        for (int j = 0; j < 8; ++j) qf[b][s][j] = (__bf16)((float)qf[b][s][j] * scale_log2);
      }
    }
  }
  const float sc = kPre ? 1.f : scale_log2;  // log2 units per unit of an MFMA score

  // A wave whose queries all lie past the group end (the last query tile of a
  // group) computes nothing, freeing its SIMD for the wave that shares it.
  const bool wave_live = w.q0 + wave * QB * 32 < w.nq;  // uniform per wave

  f32x16 o[QB][DBLK];
  RowState rs[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[b][db] = f32x16{};
    rs[b] = {0.f, 0.f};
  }

  // Two buffers (128-query items): tile t lives in buffer t % 2.  At the
  // top of each tile: wait for this wave's loads, barrier (all waves' loads
  // landed, tile t-1 fully consumed); the tile's step then starts the loads
  // of tile t+1 into the other buffer once its first K operand reads are
  // issued.
  auto begin_tile = [&](uint16_t* Kn, uint16_t* Vn, int t) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // One pass over the keys: kExpFree / kExpSub / kExpFma (softmax and P V),
  // or kStats (row maxima and sums into mx, lsum).
  constexpr int kStats = 3;
  float mx[QB], lsum[QB];
  auto run = [&](auto mode) __attribute__((always_inline)) {
    constexpr int kMode = decltype(mode)::value;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      mx[b] = -INFINITY;
      lsum[b] = 0.f;
    }
    // one tile; dma() loads later tiles after this tile's first K operand reads
    auto step = [&](uint16_t* Ks, uint16_t* Vs, int t, auto mask, uint16_t* Kn, uint16_t* Vn) {
      constexpr bool kMask = decltype(mask)::value;
      auto dma = [&]() {
        if (t + 1 < ntiles) issue(Kn, Vn, t + 1);
      };
      if (!wave_live) {  // keeps its barriers and loads, skips the math
        dma();
        return;
      }
      if constexpr (kMode == kStats) {
        dma();
        tile_stats<D, QB, kMask, Rows::kVt>(Ks, t * kBN, w.len, qf, sc, mx, lsum, lane);
      } else {
        tile_step<D, QB, kMask, Rows::kVt, kMode, !kPair>(Ks, Vs, t * kBN, w.len, qf, o, rs, scale_log2, lane, dma);
      }
    };
    using F = std::false_type;
    using T = std::true_type;
    int t = 0;
    if constexpr (kPair) {
      // tiles t, t+1 in buffers 0, 1 (t % 4 == 0) or 2, 3: at the top of
      // each pair, wait for this wave's loads, barrier, and (after the
      // pair's first K operand reads) load the next pair into the other two.
      auto pair_dma = [&](uint16_t* Ka, uint16_t* Va, uint16_t* Kb2, uint16_t* Vb2, int t0) {
        return [=, &issue]() {
          if (t0 + 2 < ntiles) issue(Ka, Va, t0 + 2);
          if (t0 + 3 < ntiles) issue(Kb2, Vb2, t0 + 3);
        };
      };
      auto sync = [&]() {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      };
      auto pstep = [&](uint16_t* Ks, uint16_t* Vs, int tt, auto mask, auto dma) {
        constexpr bool kMask = decltype(mask)::value;
        if (!wave_live) {
          dma();
          return;
        }
        if constexpr (kMode == kStats) {
          dma();
          tile_stats<D, QB, kMask, Rows::kVt>(Ks, tt * kBN, w.len, qf, sc, mx, lsum, lane);
        } else {
          tile_step<D, QB, kMask, Rows::kVt, kMode>(Ks, Vs, tt * kBN, w.len, qf, o, rs, scale_log2, lane, dma);
        }
      };
      const NoOp none{};
      for (; t + 4 <= nfull; t += 4) {
        sync();
        pstep(Ks0, Vs0, t, F{}, pair_dma(Ks2, Vs2, Ks3, Vs3, t));
        pstep(Ks1, Vs1, t + 1, F{}, none);
        sync();
        pstep(Ks2, Vs2, t + 2, F{}, pair_dma(Ks0, Vs0, Ks1, Vs1, t + 2));
        pstep(Ks3, Vs3, t + 3, F{}, none);
      }
      if (t < ntiles) {  // one to four tiles left, only the last may be partial; t % 4 == 0
        sync();
        if (t < nfull)
          pstep(Ks0, Vs0, t, F{}, pair_dma(Ks2, Vs2, Ks3, Vs3, t));
        else
          pstep(Ks0, Vs0, t, T{}, pair_dma(Ks2, Vs2, Ks3, Vs3, t));
        if (t + 1 < ntiles) {
          if (t + 1 < nfull) pstep(Ks1, Vs1, t + 1, F{}, none); else pstep(Ks1, Vs1, t + 1, T{}, none);
        }
        if (t + 2 < ntiles) {
          sync();
          if (t + 2 < nfull)
            pstep(Ks2, Vs2, t + 2, F{}, none);
          else
            pstep(Ks2, Vs2, t + 2, T{}, none);
          if (t + 3 < ntiles) pstep(Ks3, Vs3, t + 3, T{}, none);
        }
      }
      return;
    }
    for (; t + 2 <= nfull; t += 2) {
      begin_tile(Ks1, Vs1, t);
      step(Ks0, Vs0, t, F{}, Ks1, Vs1);
      begin_tile(Ks0, Vs0, t + 1);
      step(Ks1, Vs1, t + 1, F{}, Ks0, Vs0);
    }
    if (t < ntiles) {  // one or two tiles left, the last may be partial; t is even
      begin_tile(Ks1, Vs1, t);
      if (t < nfull)
        step(Ks0, Vs0, t, F{}, Ks1, Vs1);
      else
        step(Ks0, Vs0, t, T{}, Ks1, Vs1);
      if (t + 1 < ntiles) {
        begin_tile(Ks0, Vs0, t + 1);
        step(Ks1, Vs1, t + 1, T{}, Ks0, Vs0);
      }
    }
  };
  // Exponent offsets from each row's first 32 keys (key 0 always exists); a
  // wave whose rows all have those scores in [kFastLo, kFastHi] runs with no
  // offset at all.
  {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  bool free_ok = true;
  if (wave_live) {
    f32x16 s[QB];
    qk_half<D, QB>(Ks0, qf, 0, lane, s);
    if (w.len < 32) mask_half<true, QB, Rows::kVt>(s, 0, w.len, hh);
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      float m = s[b][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) m = fmaxf(m, s[b][r]);
      m = halves_max(m) * sc;
      rs[b].m_ref = m;
      free_ok &= m >= kFastLo && m <= kFastHi;
    }
  }
  if (kPre && __builtin_amdgcn_ballot_w64(!free_ok) == 0) {  // uniform per wave
#pragma unroll
    for (int b = 0; b < QB; ++b) rs[b].m_ref = 0.f;
    run(std::integral_constant<int, kExpFree>{});
  } else {
    run(std::integral_constant<int, kPre ? kExpSub : kExpFma>{});
  }

  // A denominator outside [2^-64, 2^64) or a non-finite accumulator (scores
  // far from the offset, or very large values) sends the work item to the
  // exact recomputation: row maxima and sums first, then softmax and P V
  // against max + log2(sum), which keeps every weight at most 1 and the
  // accumulator within the magnitude of the values.
  bool over = false;
  if (wave_live) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const float tot = halves_sum(rs[b].l);
      over |= !(tot < kLimit) || !(tot >= kTiny);
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) over |= !(__builtin_fabsf(o[b][db][r]) <= 3.402823466e38f);
    }
  }
  // Whether any wave must recompute.  The 128-query items with a 4,096-entry
  // key table reduce through the idle K/V buffer instead of __syncthreads_or,
  // whose 256 bytes of LDS would keep their two workgroups off one CU.
  constexpr bool kLdsTight =
      !kPair && 2 * 2 * kBN * D * 2 + tab_keys<Rows>() * 4 + kSyncOrLds > kCuLds / 2;
  bool any_over;
  if constexpr (!kLdsTight) {
    any_over = __syncthreads_or(over);
  } else {
    __syncthreads();  // every wave is past its last read of the K/V buffers
    int* const flags = reinterpret_cast<int*>(kv_lds[0]);
    if (lane == 0) flags[wave] = __builtin_amdgcn_ballot_w64(over) != 0;
    __syncthreads();
    any_over = false;
#pragma unroll
    for (int i = 0; i < NW; ++i) any_over |= flags[i] != 0;
  }
  if (any_over) {
    __syncthreads();
    issue_first();
    run(std::integral_constant<int, kStats>{});
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const auto m2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx[b]), __float_as_uint(mx[b]), false, false);
      const auto l2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum[b]), __float_as_uint(lsum[b]), false, false);
      const float m0 = __uint_as_float(m2[0]), m1 = __uint_as_float(m2[1]);
      const float mm = fmaxf(m0, m1);  // finite: key 0 lies in lane half 0
      const float ll = __uint_as_float(l2[0]) * __builtin_amdgcn_exp2f(m0 - mm) +
                       __uint_as_float(l2[1]) * __builtin_amdgcn_exp2f(m1 - mm);
      rs[b] = {mm + __log2f(ll), 0.f};
#pragma unroll
      for (int db = 0; db < DBLK; ++db) o[b][db] = f32x16{};
    }
    __syncthreads();
    issue_first();
    run(std::integral_constant<int, kPre ? kExpSub : kExpFma>{});
  }

  // ---- normalise and store: reg r of block db is channel 32*db + 8*(r/4) + 4*hh + r%4.
  // 16-byte stores where registers allow; the pair-mode kernels that read V in
  // row layout sit at the register limit and keep 8-byte ones.
  constexpr bool kWideStore = Rows::kVt || !kPair;
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float lsum = halves_sum(rs[b].l);
    const float inv = 1.0f / lsum;
    if (!qvalid[b]) continue;
    if constexpr (kEpi == kEpiPlainLse) {
      // log2 of the denominator plus the exponent offset, in natural units
      if (hh == 0) epi.lse[(int64_t)w.head * epi.n_rows + qrow[b]] = (rs[b].m_ref + __log2f(lsum)) * 0.6931471805599453f;
    }
    float scale = inv, keep = 0.f;
    int64_t orow = qrow[b];
    if constexpr (kEpi == kEpiScaled) {
      scale *= epi.alpha;
      keep = epi.beta;
    } else if constexpr (kEpi == kEpiGated) {
      orow = epi.perm[qrow[b]];
      scale *= epi.gate[orow];
      keep = epi.beta;
    } else if constexpr (kEpi == kEpiGatedInPlace) {
      scale *= epi.gate[orow];
      keep = epi.beta;
    }
    uint16_t* op = O + orow * row_stride + hoff;
    const bool acc = kEpi != kEpiPlain && keep != 0.f;  // uniform
    if constexpr (kWideStore) {
      // The lane halves hold alternating 4-channel pieces of a row; one
      // v_permlane32_swap per value pairs them up so that every lane stores 8
      // consecutive channels (16 bytes): half 0 channels 16m..16m+7 and half 1
      // channels 16m+8..16m+15 of each 16-channel run m.  An accumulating
      // epilogue loads the old values the same way, all of a row's before any
      // is used (one memory latency per row).
      u32x4 prev[DBLK][2];
      if (acc) {
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
          for (int m = 0; m < 2; ++m) prev[db][m] = *reinterpret_cast<const u32x4*>(op + 32 * db + 16 * m + 8 * hh);
      }
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float v[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[b][db][8 * m + i] * scale),
                                                             __float_as_uint(o[b][db][8 * m + 4 + i] * scale),
                                                             false, false);
            v[i] = __uint_as_float(sw[0]);
            v[4 + i] = __uint_as_float(sw[1]);
          }
          if (acc) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              v[2 * k] += keep * bf16_lo(prev[db][m][k]);
              v[2 * k + 1] += keep * bf16_hi(prev[db][m][k]);
            }
          }
          const u32x4 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7])};
          *reinterpret_cast<u32x4*>(op + 32 * db + 16 * m + 8 * hh) = pk;
        }
    } else {
      // 8 bytes per lane and store; STGA with beta != 0 (a branch summed onto
      // another) loads every old value of the row before any is used
      u32x2 prev[DBLK][4];
      if (kEpi == kEpiScaled && acc) {
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) prev[db][q4] = *reinterpret_cast<const u32x2*>(op + 32 * db + 8 * q4 + 4 * hh);
      }
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * db + 8 * q4 + 4 * hh;
          float v0 = o[b][db][4 * q4] * scale, v1 = o[b][db][4 * q4 + 1] * scale;
          float v2 = o[b][db][4 * q4 + 2] * scale, v3 = o[b][db][4 * q4 + 3] * scale;
          if (acc) {
            const u32x2 old = kEpi == kEpiScaled ? prev[db][q4] : *reinterpret_cast<const u32x2*>(op + d0);
            v0 += keep * bf16_lo(old[0]); v1 += keep * bf16_hi(old[0]);
            v2 += keep * bf16_lo(old[1]); v3 += keep * bf16_hi(old[1]);
          }
          const u32x2 pk = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          *reinterpret_cast<u32x2*>(op + d0) = pk;
        }
    }
  }
}

// One wave: groups sorted by decreasing size (ties: lower id first) and the
// prefix count of (head, query-tile) items in that order.
__global__ __launch_bounds__(kWave) void schedule_kernel(const int32_t* __restrict__ cu, int M, int H,
                                                       AttnSchedule* __restrict__ sched, int qtile = kBM) {
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
  int tiles = 0;
  if (g < M) {
    const int og = order_s[g];
    sched->order[g] = og;
    tiles = (cu[og + 1] - cu[og] + qtile - 1) / qtile * H;
  }
  // inclusive scan across the wave
  int incl = tiles;
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (g >= off) incl += v;
  }
  if (g < M) sched->prefix[g + 1] = incl;
  if (g == 0) sched->prefix[0] = 0;
}

// Window table of the shot-aware STGA, one workgroup: every shot
// [shot_start[s], shot_start[s+1]) is cut into windows of win_t frames (the
// last one shorter if needed); the shot's first window gets the previous
// shot's last `augment` frames as extra keys, its last window the next shot's
// first `augment` frames (both clipped to those shots).  Boundaries are
// clamped into [0, T] and at most max_windows entries are written, so
// malformed boundaries cannot read or write out of bounds.
constexpr int kShotThreads = 256;
__global__ __launch_bounds__(kShotThreads) void shot_windows_kernel(const int32_t* __restrict__ shot_start,
                                                                  int n_shots, int T, int win_t, int augment,
                                                                  int max_windows, ShotWindow* __restrict__ win,
                                                                  int* __restrict__ nwin) {
  __shared__ int scan[kShotThreads];
  const int tid = threadIdx.x;
  int base = 0;
  for (int s0 = 0; s0 < n_shots; s0 += kShotThreads) {
    const int s = s0 + tid;
    int lo = 0, hi = 0, cnt = 0, plo = 0, nhi = 0;
    if (s < n_shots) {
      lo = min(max(shot_start[s], 0), T);
      hi = min(max(shot_start[s + 1], lo), T);
      cnt = (hi - lo + win_t - 1) / win_t;
      plo = s > 0 ? min(max(shot_start[s - 1], 0), lo) : lo;       // previous shot's start
      nhi = s + 1 < n_shots ? min(max(shot_start[s + 2], hi), T) : hi;  // next shot's end
    }
    scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < kShotThreads; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int first = base + scan[tid] - cnt;
    for (int k = 0; k < cnt && first + k < max_windows; ++k) {
      const int t0 = lo + k * win_t;
      ShotWindow sw;
      sw.t0 = t0;
      sw.nt = min(win_t, hi - t0);
      sw.pre0 = max(plo, lo - augment);
      sw.npre = k == 0 ? lo - sw.pre0 : 0;
      sw.nxt0 = hi;
      sw.nnxt = k == cnt - 1 ? min(nhi, hi + augment) - hi : 0;
      win[first + k] = sw;
    }
    base += scan[kShotThreads - 1];
    __syncthreads();
  }
  if (tid == 0) *nwin = min(base, max_windows);
}

// Byte size of one [N, H, D] bf16 tensor if it is below 2^31 (the index-map
// windows then read rows through a buffer descriptor at 32-bit byte offsets),
// else 0.
inline uint32_t table_bytes(int64_t N, int32_t H, int32_t D) {
  const int64_t b = N * H * D * 2;
  return b < (int64_t(1) << 31) ? (uint32_t)b : 0u;
}

template <int D, class Rows, int kEpi>
int launch_attn(const void* Q, const void* K, const void* V, void* O, int64_t row_stride, float scale,
                Epilogue epi, Rows rows, int64_t items_bound, hipStream_t st) {
  const int64_t run = (int64_t)kNumXcd * kXcdRun;
  const int64_t grid = ceil_div(items_bound, run) * run;
  if (grid > 0x7fffffff) return MOGA_ERR_SHAPE;
  attn_kernel<D, kQB, Rows, kEpi><<<dim3((unsigned)grid), waves_for<Rows, kQB>() * kWave, 0, st>>>(
      static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V),
      static_cast<uint16_t*>(O), row_stride, scale * 1.4426950408889634f, epi, rows);
  MOGA_LAUNCH_CHECK();
  return MOGA_OK;
}

}  // namespace
}  // namespace moga

extern "C" int moga_group_attention(const void* Qp, const void* Kp, const void* Vp, const int32_t* cu_seqlens,
                                    int64_t N, int32_t H, int32_t D, int32_t M, float softmax_scale, void* Op,
                                    void* ws, size_t ws_bytes, void* stream) {
  using namespace moga;
  if (!Qp || !Kp || !Vp || !cu_seqlens || !Op) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1 || H < 1 || D < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups || !valid_head_dims(H, D)) return MOGA_ERR_UNSUPPORTED;
  const size_t need = moga_workspace_bytes(MOGA_OP_GROUP_ATTENTION, N, M, H, D);
  if (!ws || ws_bytes < need) return MOGA_ERR_WORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  hipStream_t st = as_stream(stream);
  auto* sched = static_cast<AttnSchedule*>(ws);
  schedule_kernel<<<1, kWave, 0, st>>>(cu_seqlens, M, H, sched);
  MOGA_LAUNCH_CHECK();
  MogaRows rows{cu_seqlens, sched, M, H};
  const int64_t bound = (ceil_div(N, kBM) + M) * H;
  const Epilogue epi{1.f, 0.f, nullptr, nullptr, nullptr, 0};
  if (D == 128) return launch_attn<128, MogaRows, kEpiPlain>(Qp, Kp, Vp, Op, (int64_t)H * D, scale, epi, rows, bound, st);
  return launch_attn<64, MogaRows, kEpiPlain>(Qp, Kp, Vp, Op, (int64_t)H * D, scale, epi, rows, bound, st);
}

extern "C" int moga_stga_attention(const void* Q, const void* K, const void* V, int32_t T, int32_t Hs, int32_t Ws,
                                   int32_t win_t, int32_t tile_h, int32_t tile_w, int32_t H, int32_t D,
                                   float softmax_scale, float alpha, float beta, void* O, void* ws,
                                   size_t ws_bytes, void* stream) {
  using namespace moga;
  (void)ws;  // static windows need no workspace (moga_workspace_bytes(MOGA_OP_STGA_ATTENTION, ...) == 0)
  (void)ws_bytes;
  if (!Q || !K || !V || !O) return MOGA_ERR_NULL;
  if (T < 1 || Hs < 1 || Ws < 1 || win_t < 1 || tile_h < 1 || tile_w < 1 || H < 1 || D < 1) return MOGA_ERR_SHAPE;
  if (T % win_t || Hs % tile_h || Ws % tile_w) return MOGA_ERR_SHAPE;
  const int64_t N = (int64_t)T * Hs * Ws;
  const int64_t gsize = (int64_t)win_t * tile_h * tile_w;
  if (N >= (int64_t(1) << 31)) return MOGA_ERR_SHAPE;
  if (gsize > (int64_t(1) << 20) || !valid_head_dims(H, D)) return MOGA_ERR_UNSUPPORTED;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  const int tpg = (int)ceil_div(gsize, StgaRows::kQueries);
  const int64_t items = (N / gsize) * H * tpg;
  if (items > 0x7fffffff) return MOGA_ERR_SHAPE;
  StgaRows rows{Hs, Ws, win_t, tile_h, tile_w, Hs / tile_h, Ws / tile_w, tpg, H, (int)items, table_bytes(N, H, D),
                1.0f / (float)(tile_h * tile_w), 1.0f / (float)tile_w};
  hipStream_t st = as_stream(stream);
  const Epilogue epi{alpha, beta, nullptr, nullptr, nullptr, 0};
  if (D == 128) return launch_attn<128, StgaRows, kEpiScaled>(Q, K, V, O, (int64_t)H * D, scale, epi, rows, items, st);
  return launch_attn<64, StgaRows, kEpiScaled>(Q, K, V, O, (int64_t)H * D, scale, epi, rows, items, st);
}

extern "C" int moga_group_attention_unpermute(const void* Qp, const void* Kp, const void* Vp,
                                              const int32_t* cu_seqlens, const int32_t* perm, const float* gate,
                                              int64_t N, int32_t H, int32_t D, int32_t M, float softmax_scale,
                                              float beta, void* O, void* ws, size_t ws_bytes, void* stream) {
  using namespace moga;
  if (!Qp || !Kp || !Vp || !cu_seqlens || !perm || !gate || !O) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1 || H < 1 || D < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups || !valid_head_dims(H, D)) return MOGA_ERR_UNSUPPORTED;
  const size_t need = moga_workspace_bytes(MOGA_OP_GROUP_ATTENTION, N, M, H, D);
  if (!ws || ws_bytes < need) return MOGA_ERR_WORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  hipStream_t st = as_stream(stream);
  auto* sched = static_cast<AttnSchedule*>(ws);
  schedule_kernel<<<1, kWave, 0, st>>>(cu_seqlens, M, H, sched);
  MOGA_LAUNCH_CHECK();
  MogaRows rows{cu_seqlens, sched, M, H};
  const int64_t bound = (ceil_div(N, kBM) + M) * H;
  const Epilogue epi{1.f, beta, perm, gate, nullptr, 0};
  if (D == 128) return launch_attn<128, MogaRows, kEpiGated>(Qp, Kp, Vp, O, (int64_t)H * D, scale, epi, rows, bound, st);
  return launch_attn<64, MogaRows, kEpiGated>(Qp, Kp, Vp, O, (int64_t)H * D, scale, epi, rows, bound, st);
}

extern "C" int moga_group_attention_unpermute_vt(const void* Qp, const void* Kp, const void* Vt,
                                                 const int32_t* cu_seqlens, const int32_t* perm, const float* gate,
                                                 int64_t N, int32_t H, int32_t D, int32_t M, float softmax_scale,
                                                 float beta, void* O, void* ws, size_t ws_bytes, void* stream) {
  using namespace moga;
  if (!Qp || !Kp || !Vt || !cu_seqlens || !perm || !gate || !O) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1 || H < 1 || D < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups || !valid_head_dims(H, D) || N > kVtMaxTokens) return MOGA_ERR_UNSUPPORTED;
  const size_t need = moga_workspace_bytes(MOGA_OP_GROUP_ATTENTION, N, M, H, D);
  if (!ws || ws_bytes < need) return MOGA_ERR_WORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  hipStream_t st = as_stream(stream);
  auto* sched = static_cast<AttnSchedule*>(ws);
  schedule_kernel<<<1, kWave, 0, st>>>(cu_seqlens, M, H, sched);
  MOGA_LAUNCH_CHECK();
  MogaVtRows rows{MogaRows{cu_seqlens, sched, M, H}, vt_row_length(N)};
  const int64_t bound = (ceil_div(N, kBM) + M) * H;
  const Epilogue epi{1.f, beta, perm, gate, nullptr, 0};
  if (D == 128) return launch_attn<128, MogaVtRows, kEpiGated>(Qp, Kp, Vt, O, (int64_t)H * D, scale, epi, rows, bound, st);
  return launch_attn<64, MogaVtRows, kEpiGated>(Qp, Kp, Vt, O, (int64_t)H * D, scale, epi, rows, bound, st);
}

extern "C" int moga_group_attention_unpermute_vtq(const void* Q, const void* Kp, const void* Vt,
                                                  const int32_t* cu_seqlens, const int32_t* perm, const float* gate,
                                                  int64_t N, int32_t H, int32_t D, int32_t M, float softmax_scale,
                                                  float beta, void* O, void* ws, size_t ws_bytes, void* stream) {
  using namespace moga;
  if (!Q || !Kp || !Vt || !cu_seqlens || !perm || !gate || !O) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1 || H < 1 || D < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups || !valid_head_dims(H, D) || N > kVtMaxTokens) return MOGA_ERR_UNSUPPORTED;
  const size_t need = moga_workspace_bytes(MOGA_OP_GROUP_ATTENTION, N, M, H, D);
  if (!ws || ws_bytes < need) return MOGA_ERR_WORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  hipStream_t st = as_stream(stream);
  auto* sched = static_cast<AttnSchedule*>(ws);
  // Groups of fewer than kShortGroup tokens on average take 128-query items.
  const bool short_groups = N < (int64_t)kShortGroup * M;
  const int qtile = short_groups ? MogaVtQRows128::kQueries : kBM;
  schedule_kernel<<<1, kWave, 0, st>>>(cu_seqlens, M, H, sched, qtile);
  MOGA_LAUNCH_CHECK();
  MogaVtQRows128 rows;
  rows.base = MogaRows{cu_seqlens, sched, M, H};
  rows.ldv = vt_row_length(N);
  rows.perm = perm;
  const int64_t bound = (ceil_div(N, qtile) + M) * H;
  const Epilogue epi{1.f, beta, nullptr, gate, nullptr, 0};
  const MogaVtQRows& rows256 = rows;
  if (short_groups) {
    if (D == 128)
      return launch_attn<128, MogaVtQRows128, kEpiGatedInPlace>(Q, Kp, Vt, O, (int64_t)H * D, scale, epi, rows, bound,
                                                                st);
    return launch_attn<64, MogaVtQRows128, kEpiGatedInPlace>(Q, Kp, Vt, O, (int64_t)H * D, scale, epi, rows, bound, st);
  }
  if (D == 128)
    return launch_attn<128, MogaVtQRows, kEpiGatedInPlace>(Q, Kp, Vt, O, (int64_t)H * D, scale, epi, rows256, bound,
                                                           st);
  return launch_attn<64, MogaVtQRows, kEpiGatedInPlace>(Q, Kp, Vt, O, (int64_t)H * D, scale, epi, rows256, bound, st);
}

extern "C" size_t moga_stga_shot_workspace_bytes(int32_t T, int32_t n_shots, int32_t win_t) {
  if (T < 1 || n_shots < 1 || win_t < 1) return 0;
  const int64_t max_windows = moga::ceil_div(T, win_t) + n_shots;
  return 256 + (size_t)max_windows * sizeof(moga::ShotWindow);
}

extern "C" int moga_stga_shot_attention(const void* Q, const void* K, const void* V, int32_t T, int32_t Hs,
                                        int32_t Ws, const int32_t* shot_start, int32_t n_shots, int32_t win_t,
                                        int32_t tile_h, int32_t tile_w, int32_t augment, int32_t H, int32_t D,
                                        float softmax_scale, float alpha, float beta, void* O, void* ws,
                                        size_t ws_bytes, void* stream) {
  using namespace moga;
  if (!Q || !K || !V || !O || !shot_start) return MOGA_ERR_NULL;
  if (T < 1 || Hs < 1 || Ws < 1 || n_shots < 1 || win_t < 1 || tile_h < 1 || tile_w < 1 || H < 1 || D < 1)
    return MOGA_ERR_SHAPE;
  if (n_shots > T || Hs % tile_h || Ws % tile_w) return MOGA_ERR_SHAPE;
  const int64_t N = (int64_t)T * Hs * Ws;
  const int64_t area = (int64_t)tile_h * tile_w;
  if (N >= (int64_t(1) << 31)) return MOGA_ERR_SHAPE;
  if (augment < 0 || augment > 64) return MOGA_ERR_SHAPE;
  if ((int64_t)(win_t + 2 * augment) * area > (int64_t(1) << 20) || !valid_head_dims(H, D)) return MOGA_ERR_UNSUPPORTED;
  const size_t need = moga_stga_shot_workspace_bytes(T, n_shots, win_t);
  if (!ws || ws_bytes < need) return MOGA_ERR_WORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  const int max_windows = (int)(ceil_div(T, win_t) + n_shots);
  const int tpg = (int)ceil_div((int64_t)win_t * area, ShotRows::kQueries);
  const int ntx = Ws / tile_w, nspatial = (Hs / tile_h) * ntx;
  const int64_t items = (int64_t)max_windows * nspatial * H * tpg;
  if (items > 0x7fffffff) return MOGA_ERR_SHAPE;
  hipStream_t st = as_stream(stream);
  int* nwin = static_cast<int*>(ws);
  auto* win = reinterpret_cast<ShotWindow*>(static_cast<char*>(ws) + 256);
  shot_windows_kernel<<<1, kShotThreads, 0, st>>>(shot_start, n_shots, T, win_t, augment, max_windows, win, nwin);
  MOGA_LAUNCH_CHECK();
  ShotRows rows{win, nwin, Hs, Ws, tile_h, tile_w, ntx, nspatial, tpg, H, table_bytes(N, H, D),
                1.0f / (float)(tile_h * tile_w), 1.0f / (float)tile_w};
  const Epilogue epi{alpha, beta, nullptr, nullptr, nullptr, 0};
  if (D == 128) return launch_attn<128, ShotRows, kEpiScaled>(Q, K, V, O, (int64_t)H * D, scale, epi, rows, items, st);
  return launch_attn<64, ShotRows, kEpiScaled>(Q, K, V, O, (int64_t)H * D, scale, epi, rows, items, st);
}

extern "C" int moga_group_attention_fused(const void* Q, const void* K, const void* V, const int32_t* cu_seqlens,
                                          const int32_t* perm, const float* gate, int64_t N, int32_t H, int32_t D,
                                          int32_t M, float softmax_scale, float beta, void* O, void* ws,
                                          size_t ws_bytes, void* stream) {
  using namespace moga;
  if (!Q || !K || !V || !cu_seqlens || !perm || !gate || !O) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1 || H < 1 || D < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups || !valid_head_dims(H, D)) return MOGA_ERR_UNSUPPORTED;
  const size_t need = moga_workspace_bytes(MOGA_OP_GROUP_ATTENTION, N, M, H, D);
  if (!ws || ws_bytes < need) return MOGA_ERR_WORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  hipStream_t st = as_stream(stream);
  auto* sched = static_cast<AttnSchedule*>(ws);
  schedule_kernel<<<1, kWave, 0, st>>>(cu_seqlens, M, H, sched);
  MOGA_LAUNCH_CHECK();
  MogaPermRows rows{MogaRows{cu_seqlens, sched, M, H}, perm};
  const int64_t bound = (ceil_div(N, kBM) + M) * H;
  const Epilogue epi{1.f, beta, nullptr, gate, nullptr, 0};
  if (D == 128)
    return launch_attn<128, MogaPermRows, kEpiGatedInPlace>(Q, K, V, O, (int64_t)H * D, scale, epi, rows, bound, st);
  return launch_attn<64, MogaPermRows, kEpiGatedInPlace>(Q, K, V, O, (int64_t)H * D, scale, epi, rows, bound, st);
}

extern "C" int moga_group_attention_train(const void* Qp, const void* Kp, const void* Vp, const int32_t* cu_seqlens,
                                          int64_t N, int32_t H, int32_t D, int32_t M, float softmax_scale, void* Op,
                                          float* lse, void* ws, size_t ws_bytes, void* stream) {
  using namespace moga;
  if (!Qp || !Kp || !Vp || !cu_seqlens || !Op || !lse) return MOGA_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1 || H < 1 || D < 1) return MOGA_ERR_SHAPE;
  if (M > kMaxGroups || !valid_head_dims(H, D)) return MOGA_ERR_UNSUPPORTED;
  const size_t need = moga_workspace_bytes(MOGA_OP_GROUP_ATTENTION, N, M, H, D);
  if (!ws || ws_bytes < need) return MOGA_ERR_WORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  hipStream_t st = as_stream(stream);
  auto* sched = static_cast<AttnSchedule*>(ws);
  schedule_kernel<<<1, kWave, 0, st>>>(cu_seqlens, M, H, sched);
  MOGA_LAUNCH_CHECK();
  MogaRows rows{cu_seqlens, sched, M, H};
  const int64_t bound = (ceil_div(N, kBM) + M) * H;
  const Epilogue epi{1.f, 0.f, nullptr, nullptr, lse, N};
  if (D == 128) return launch_attn<128, MogaRows, kEpiPlainLse>(Qp, Kp, Vp, Op, (int64_t)H * D, scale, epi, rows, bound, st);
  return launch_attn<64, MogaRows, kEpiPlainLse>(Qp, Kp, Vp, Op, (int64_t)H * D, scale, epi, rows, bound, st);
}
