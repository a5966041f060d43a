// Host-only entry points of libmoga: workspace sizing, status strings, version.
#include "moga_internal.h"

extern "C" size_t moga_workspace_bytes(int32_t op, int64_t N, int32_t M, int32_t H, int32_t D) {
  using namespace moga;
  (void)H;
  if (N < 1 || N >= (int64_t(1) << 31) || M < 1 || M > kMaxGroups) return 0;
  switch (op) {
    case MOGA_OP_PERMUTE:  // per-(group, block) counts and base offsets
      return align_up(2 * (size_t)M * (size_t)sort_blocks(N) * sizeof(int32_t), 256);
    case MOGA_OP_GROUP_ATTENTION:  // the largest-group-first schedule
      return align_up(sizeof(AttnSchedule), 256);
    case MOGA_OP_BALANCE_STATS:  // per-(group, block) counts and gate sums
      return align_up(2 * (size_t)M * (size_t)sort_blocks(N) * 4, 256);
    case MOGA_OP_ATTENTION_BACKWARD:  // two largest-group-first schedules (key and query tiles)
      return 2048;
    case MOGA_OP_ROUTE_BACKWARD: {  // dlogits [N, M], dW_r block partials, db block partials
      if (D < 1) return 0;
      const size_t nblk = (size_t)ceil_div(N, 1024);
      return align_up((size_t)N * M * 4, 256) + align_up(nblk * M * (size_t)D * 4, 256) + align_up(nblk * M * 4, 256);
    }
    default:
      return 0;
  }
}

extern "C" const char* moga_strerror(int32_t status) {
  switch (status) {
    case MOGA_OK: return "success";
    case MOGA_ERR_NULL: return "a required pointer is NULL";
    case MOGA_ERR_SHAPE: return "a size is out of range or sizes disagree";
    case MOGA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOGA_ERR_WORKSPACE: return "workspace missing or too small";
    case MOGA_ERR_HIP: return "HIP runtime refused a launch";
    default: return "unknown status";
  }
}

// 0.2.0: shot-aware STGA, gather on load, backward pass
// 0.3.0: transposed-V gather and attention (moga_permute_vt, moga_group_attention_unpermute_vt)
// 0.3.1: queries read through perm (moga_group_attention_unpermute_vtq; moga_permute_vt without Q)
// 0.4.0: moga_route and moga_stga_attention take (ws, ws_bytes) like the other steps
extern "C" int32_t moga_version(void) { return 410; }
