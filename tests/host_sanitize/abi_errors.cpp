// Host-side argument checking of every libmoga entry point, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the
// device code is compiled as usual and never launched: every call below has
// one invalid argument, which must be reported before any launch).  Also
// sweeps the workspace-size functions over extreme sizes, where an integer
// overflow would be undefined behaviour.  Exit status = number of failures.
#include <cstdint>
#include <cstdio>

#include "moga.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  // stand-ins for device buffers: host checks must not dereference them
  void* P = reinterpret_cast<void*>(uintptr_t(0x1000));
  auto* I = static_cast<int32_t*>(P);
  auto* F = static_cast<float*>(P);
  const size_t big = size_t(1) << 40;  // "enough" workspace
  const int64_t N = 1000;

  expect(moga_route(nullptr, P, nullptr, N, 64, 4, I, F, nullptr, 0, nullptr), MOGA_ERR_NULL, "route X");
  expect(moga_route(P, P, nullptr, 0, 64, 4, I, F, nullptr, 0, nullptr), MOGA_ERR_SHAPE, "route N");
  expect(moga_route(P, P, nullptr, N, 64, 65, I, F, nullptr, 0, nullptr), MOGA_ERR_UNSUPPORTED, "route M");

  expect(moga_permute(nullptr, P, P, P, N, 2, 128, 4, P, P, P, I, I, I, P, big, nullptr), MOGA_ERR_NULL,
         "permute group_id");
  expect(moga_permute(I, P, P, nullptr, N, 2, 128, 4, P, P, P, I, I, I, P, big, nullptr), MOGA_ERR_NULL,
         "permute V alone missing");
  expect(moga_permute(I, P, P, P, N, 2, 96, 4, P, P, P, I, I, I, P, big, nullptr), MOGA_ERR_UNSUPPORTED,
         "permute D");
  expect(moga_permute(I, P, P, P, N, 2, 128, 4, P, P, P, I, I, I, P, 0, nullptr), MOGA_ERR_WORKSPACE,
         "permute ws");

  expect(moga_permute_vt(I, P, P, P, N, 2, 128, 4, nullptr, P, P, I, I, I, P, big, nullptr), MOGA_ERR_NULL,
         "permute_vt Q without Qp");
  expect(moga_permute_vt(I, P, P, P, (int64_t(1) << 23), 2, 128, 4, P, P, P, I, I, I, P, big, nullptr),
         MOGA_ERR_UNSUPPORTED, "permute_vt N");
  expect(moga_permute_vt_noalloc(I, P, P, P, N, 2, 128, 4, nullptr, P, P, I, I, I, nullptr), MOGA_ERR_NULL,
         "permute_vt_noalloc Q without Qp");
  expect(moga_permute_vt_noalloc(I, nullptr, P, P, (int64_t(1) << 21) + 1024, 2, 128, 64, nullptr, P, P, I, I, I,
                                 nullptr),
         MOGA_ERR_WORKSPACE, "permute_vt_noalloc beyond its scratch");

  expect(moga_group_attention(P, P, P, I, N, 2, 128, 4, 0.f, P, P, 0, nullptr), MOGA_ERR_WORKSPACE,
         "attention ws");
  expect(moga_group_attention(P, P, P, I, N, 2, 128, 0, 0.f, P, P, big, nullptr), MOGA_ERR_SHAPE, "attention M");
  expect(moga_group_attention(P, P, P, I, N, 65, 128, 4, 0.f, P, P, big, nullptr), MOGA_ERR_UNSUPPORTED,
         "attention H*D");

  expect(moga_group_attention_unpermute(P, P, P, I, nullptr, F, N, 2, 128, 4, 0.f, 0.f, P, P, big, nullptr),
         MOGA_ERR_NULL, "attention_unpermute perm");
  expect(moga_group_attention_unpermute_vt(P, P, P, I, I, F, -5, 2, 128, 4, 0.f, 0.f, P, P, big, nullptr),
         MOGA_ERR_SHAPE, "attention_unpermute_vt N");
  expect(moga_group_attention_unpermute_vtq(P, P, P, I, I, F, N, 2, 64, 4, 0.f, 0.f, nullptr, P, big, nullptr),
         MOGA_ERR_NULL, "attention_unpermute_vtq O");
  expect(moga_group_attention_fused(P, P, P, I, I, F, N, 2, 32, 4, 0.f, 0.f, P, P, big, nullptr),
         MOGA_ERR_UNSUPPORTED, "attention_fused D");

  expect(moga_unpermute(P, I, nullptr, N, 2, 128, 0.f, P, nullptr), MOGA_ERR_NULL, "unpermute gate");
  expect(moga_stga_attention(P, P, P, 5, 30, 52, 3, 30, 26, 2, 128, 0.f, 1.f, 0.f, P, nullptr, 0, nullptr), MOGA_ERR_SHAPE,
         "stga win_t does not divide T");
  expect(moga_stga_attention(P, P, P, 6, 30, 52, 3, 30, 26, 2, 128, 0.f, 1.f, 0.f, nullptr, nullptr, 0, nullptr),
         MOGA_ERR_NULL, "stga O");
  expect(moga_stga_shot_attention(P, P, P, 6, 30, 52, I, 0, 3, 30, 26, 1, 2, 128, 0.f, 1.f, 0.f, P, P, big,
                                  nullptr),
         MOGA_ERR_SHAPE, "stga_shot no shots");
  expect(moga_balance_stats(I, F, N, 4, 0.1f, F, F, F, P, 0, nullptr), MOGA_ERR_WORKSPACE, "balance ws");
  expect(moga_group_attention_train(P, P, P, I, N, 2, 128, 4, 0.f, P, nullptr, P, big, nullptr), MOGA_ERR_NULL,
         "train lse");
  expect(moga_unpermute_backward(P, P, I, F, N, 2, 100, P, F, F, nullptr), MOGA_ERR_UNSUPPORTED,
         "unpermute_backward D");
  expect(moga_group_attention_backward(P, P, P, P, F, F, I, I, N, 2, 128, 4, 0.f, P, P, P, P, 0, nullptr),
         MOGA_ERR_WORKSPACE, "attention_backward ws");
  expect(moga_route_backward(P, P, nullptr, I, F, N, 48, 4, F, F, F, P, big, nullptr), MOGA_ERR_UNSUPPORTED,
         "route_backward d_model");

  // workspace sizes at the extremes of the supported ranges (no overflow, no UB)
  const int64_t Ns[] = {1, 1000, (int64_t(1) << 31) - 1};
  const int32_t Ms[] = {1, 64}, Hs[] = {1, 64}, Ds[] = {64, 128};
  size_t sum = 0;
  for (int op = 0; op <= MOGA_OP_ATTENTION_BACKWARD; ++op)
    for (int64_t n : Ns)
      for (int32_t m : Ms)
        for (int32_t h : Hs)
          for (int32_t d : Ds) sum += moga_workspace_bytes(op, n, m, h, d) & 1;
  sum += moga_stga_shot_workspace_bytes(0x7fffffff, 0x7fffffff, 1) & 1;
  sum += moga_stga_shot_workspace_bytes(1, 1, 1) & 1;
  for (int s = -6; s <= 0; ++s) sum += moga_strerror(s)[0] != 0;
  std::printf("checked %s, version %d, %zu\n", failures ? "with failures" : "ok", moga_version(), sum);
  return failures;
}
