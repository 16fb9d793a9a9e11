// Host-side driver for the sanitizer build of libsqa (ASan + UBSan on the
// host code, device code unchanged). It calls every C-ABI entry point with
// arguments that validation must reject -- null, misaligned or overlapping
// pointers, bad shapes, unsupported head dims, sizes past the kernels'
// launch limits, short workspaces -- plus zero-sized no-ops and the size
// queries at extreme values. Pointers are fake addresses that are never
// dereferenced: no call here reaches a kernel launch, so it runs on hosts
// without a GPU. Exit status 0 when every status matches; the sanitizers
// abort on any finding.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "sqa.h"

namespace {

int g_fail = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: status %d (%s), expected %d; last error: %s\n", what, got, sqa_status_str(got), want,
                sqa_last_error());
    ++g_fail;
  }
  if (want != SQA_OK && std::strlen(sqa_last_error()) == 0) {
    std::printf("FAIL %s: no error detail\n", what);
    ++g_fail;
  }
}

void* fake(int i) { return reinterpret_cast<void*>(uintptr_t(0x10000) + uintptr_t(i) * (uintptr_t(1) << 40)); }
void* fake_near(int i) { return reinterpret_cast<void*>(uintptr_t(0x10000) + uintptr_t(i) * 0x100000); }
char* cfake(int i) { return static_cast<char*>(fake(i)); }
const int32_t* ifake(int i) { return static_cast<const int32_t*>(fake(i)); }

void attn_forward() {
  // shape, head, dtype and argument rules
  expect(sqa_attn_fwd(nullptr, fake(1), fake(2), fake(3), 1, 8, 4, 1024, 64, SQA_BF16, 0.125f, 0, nullptr, nullptr),
         SQA_ERR_NULL, "fwd null q");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), 1, 8, 9, 1024, 64, SQA_BF16, 0.125f, 0, nullptr, nullptr),
         SQA_ERR_SHAPE, "fwd H_kv > H_q");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), -1, 8, 4, 1024, 64, SQA_BF16, 0.125f, 0, nullptr, nullptr),
         SQA_ERR_SHAPE, "fwd negative B");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), 1, 8, 4, INT64_MAX, 64, SQA_BF16, 0.125f, 0, nullptr,
                      nullptr),
         SQA_ERR_SHAPE, "fwd huge N");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), INT64_MAX, INT64_MAX, 1, 1, 64, SQA_BF16, 0.125f, 0,
                      nullptr, nullptr),
         SQA_ERR_SHAPE, "fwd huge B and H_q");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), 1, 8, 4, 1024, 48, SQA_BF16, 0.125f, 0, nullptr, nullptr),
         SQA_ERR_UNSUPPORTED, "fwd d = 48");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), 1, 8, 4, 1024, 64, 9, 0.125f, 0, nullptr, nullptr),
         SQA_ERR_UNSUPPORTED, "fwd dtype");
  expect(sqa_attn_fwd(cfake(0) + 8, fake(1), fake(2), fake(3), 1, 8, 4, 1024, 64, SQA_BF16, 0.125f, 0, nullptr,
                      nullptr),
         SQA_ERR_ALIGN, "fwd misaligned q");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), 1, 8, 4, 1024, 64, SQA_BF16, 1.0f / 0.0f, 0, nullptr,
                      nullptr),
         SQA_ERR_ARG, "fwd scale inf");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(0), 1, 8, 4, 1024, 64, SQA_BF16, 0.125f, 0, nullptr, nullptr),
         SQA_ERR_ARG, "fwd o aliases q");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), 1, 8, 4, 1024, 64, SQA_BF16, 0.125f, 2, nullptr, nullptr),
         SQA_ERR_ARG, "fwd causal = 2");
  // launch limits
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), 1, 8, 4, int64_t(1) << 24, 64, SQA_BF16, 0.125f, 0,
                      nullptr, nullptr),
         SQA_ERR_SHAPE, "fwd d=64 N = 2^24");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), 1, 8, 4, int64_t(1) << 23, 128, SQA_BF16, 0.125f, 1,
                      nullptr, nullptr),
         SQA_ERR_SHAPE, "fwd d=128 N = 2^23");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), int64_t(1) << 31, 1, 1, 1, 16, SQA_BF16, 0.125f, 0,
                      nullptr, nullptr),
         SQA_ERR_SHAPE, "fwd B * H_kv = 2^31");
  expect(sqa_attn_fwd(fake(0), fake(1), fake(2), fake(3), int64_t(1) << 31, 1, 1, 1, 16, SQA_F32, 0.125f, 0, nullptr,
                      nullptr),
         SQA_ERR_SHAPE, "fwd fp32 grid");
  // zero-sized problems
  expect(sqa_attn_fwd(nullptr, nullptr, nullptr, nullptr, 0, 8, 4, 1024, 64, SQA_BF16, 0.125f, 0, nullptr, nullptr),
         SQA_OK, "fwd B = 0");
  // splits
  expect(sqa_attn_fwd_split(fake(0), fake(1), fake(2), fake(3), 1, 8, 4, 4096, 64, SQA_BF16, 0.125f, 0, nullptr, 2,
                            nullptr, 0, nullptr),
         SQA_ERR_WORKSPACE, "split without workspace");
  expect(sqa_attn_fwd_split(fake(0), fake(1), fake(2), fake(3), 1, 8, 4, 4096, 64, SQA_BF16, 0.125f, 0, nullptr, 17,
                            fake(4), 1 << 30, nullptr),
         SQA_ERR_ARG, "split count 17");
  expect(sqa_attn_fwd_split(fake(0), fake(1), fake(2), fake(3), 1, 8, 4, 4096, 64, SQA_F32, 0.125f, 0, nullptr, 2,
                            fake(4), 1 << 30, nullptr),
         SQA_ERR_UNSUPPORTED, "split fp32");
  expect(sqa_attn_fwd_split(fake(0), fake(1), fake(2), fake(3), 1, 8, 4, 4096, 64, SQA_BF16, 0.125f, 0, nullptr, 2,
                            fake(1), size_t(1) << 30, nullptr),
         SQA_ERR_ARG, "split workspace aliases k");
  // packed batches
  expect(sqa_attn_fwd_varlen(fake(0), fake(1), fake(2), fake(3), nullptr, 4, 8, 4, 4096, 2048, 64, SQA_BF16, 0.125f,
                             1, nullptr, nullptr),
         SQA_ERR_NULL, "varlen null cu");
  expect(sqa_attn_fwd_varlen(fake(0), fake(1), fake(2), fake(3), ifake(4), 4, 8, 4, 4096, 5000, 64, SQA_BF16, 0.125f,
                             1, nullptr, nullptr),
         SQA_ERR_SHAPE, "varlen max_seqlen > T");
  expect(sqa_attn_fwd_varlen(fake(0), fake(1), fake(2), fake(3), reinterpret_cast<const int32_t*>(cfake(4) + 2), 4, 8, 4, 4096, 2048, 64, SQA_BF16,
                             0.125f, 1, nullptr, nullptr),
         SQA_ERR_ALIGN, "varlen misaligned cu");
  expect(sqa_attn_fwd_varlen(fake(0), fake(1), fake(2), fake(3), ifake(4), 1, 8, 4, int64_t(1) << 24, int64_t(1) << 24,
                             64, SQA_BF16, 0.125f, 0, nullptr, nullptr),
         SQA_ERR_SHAPE, "varlen d=64 launch limit");
  // tail split (the plan assumes 256 CUs without a device)
  expect(sqa_attn_fwd_tail(fake(0), fake(1), fake(2), fake(3), 1, 4, 4, 200000, 64, SQA_BF16, 0.125f, 0, nullptr,
                           nullptr, 0, nullptr),
         SQA_ERR_WORKSPACE, "tail without workspace");
  expect(sqa_attn_fwd_tail(fake(0), fake(1), fake(2), fake(3), 1, 4, 4, 200000, 64, SQA_BF16, 0.125f, 0, nullptr,
                           fake(2), size_t(1) << 30, nullptr),
         SQA_ERR_ARG, "tail workspace aliases v");
  expect(sqa_attn_fwd_tail(fake(0), fake(1), fake(2), fake(3), 1, 4, 0, 200000, 64, SQA_BF16, 0.125f, 0, nullptr,
                           fake(4), size_t(1) << 30, nullptr),
         SQA_ERR_SHAPE, "tail H_kv = 0");
  expect(sqa_attn_fwd_varlen_split(fake(0), fake(1), fake(2), fake(3), ifake(4), 4, 8, 4, 4096, 2048, 64, SQA_BF16,
                                   0.125f, 0, nullptr, 2, fake(4), size_t(1) << 30, nullptr),
         SQA_ERR_ARG, "varlen split workspace aliases cu");
}

void attn_backward() {
  expect(sqa_attn_bwd(fake(0), fake(1), fake(2), fake(3), fake(4), nullptr, fake(6), fake(7), fake(8), 1, 8, 4,
                      1024, 64, SQA_BF16, 0.125f, 0, fake(9), 1 << 20, nullptr),
         SQA_ERR_NULL, "bwd null lse");
  expect(sqa_attn_bwd(fake(0), fake(1), fake(2), fake(3), fake(4), static_cast<const float*>(fake(5)), fake(6),
                      fake(7), fake(8), 1, 8, 4, 1024, 16, SQA_BF16, 0.125f, 0, fake(9), 1 << 20, nullptr),
         SQA_ERR_UNSUPPORTED, "bwd d = 16");
  expect(sqa_attn_bwd(fake(0), fake(1), fake(2), fake(3), fake(4), static_cast<const float*>(fake(5)), fake(6),
                      fake(7), fake(8), 1, 8, 4, 1024, 64, SQA_BF16, 0.125f, 0, fake(9), 100, nullptr),
         SQA_ERR_WORKSPACE, "bwd short workspace");
  expect(sqa_attn_bwd(fake(0), fake(1), fake(2), fake(3), fake(4), static_cast<const float*>(fake(5)), fake(3),
                      fake(7), fake(8), 1, 8, 4, 1024, 64, SQA_BF16, 0.125f, 0, fake(9), 1 << 20, nullptr),
         SQA_ERR_ARG, "bwd dq aliases o");
  expect(sqa_attn_bwd(fake(0), fake(1), fake(2), fake(3), fake(4), static_cast<const float*>(fake(5)), fake(6),
                      fake(7), fake(8), 1, 8, 4, int64_t(1) << 24, 64, SQA_BF16, 0.125f, 0, fake(9),
                      size_t(1) << 36, nullptr),
         SQA_ERR_SHAPE, "bwd d=64 launch limit");
  expect(sqa_attn_bwd_split(fake(0), fake(1), fake(2), fake(3), fake(4), static_cast<const float*>(fake(5)), fake(6),
                            fake(7), fake(8), 1, 8, 4, 4096, 64, SQA_BF16, 0.125f, 1, 2, fake(9), size_t(1) << 36,
                            nullptr),
         SQA_ERR_UNSUPPORTED, "bwd split causal");
  expect(sqa_attn_bwd_noalloc(fake(0), fake(1), fake(2), fake(3), fake(4), static_cast<const float*>(fake(5)),
                              fake(6), fake(7), fake(8), 1, 32, 8, 262144, 64, SQA_BF16, 0.125f, 0, nullptr),
         SQA_ERR_WORKSPACE, "bwd noalloc over its buffer");
  expect(sqa_attn_bwd_noalloc(fake(0), fake(1), fake(2), fake(3), fake(4), static_cast<const float*>(fake(5)),
                              fake(6), fake(7), fake(8), 1, 8, 9, 1024, 64, SQA_BF16, 0.125f, 0, nullptr),
         SQA_ERR_SHAPE, "bwd noalloc H_kv > H_q");
  expect(sqa_attn_bwd_varlen(fake(0), fake(1), fake(2), fake(3), fake(4), static_cast<const float*>(fake(5)), fake(6),
                             fake(7), fake(8), nullptr, 4, 8, 4, 4096, 2048, 64, SQA_BF16, 0.125f, 1, fake(9),
                             size_t(1) << 30, nullptr),
         SQA_ERR_NULL, "bwd varlen null cu");
  expect(sqa_attn_bwd_varlen_split(fake(0), fake(1), fake(2), fake(3), fake(4), static_cast<const float*>(fake(5)),
                                   fake(6), fake(7), fake(8), ifake(10), 4, 8, 4, 4096, 2048, 64, SQA_BF16, 0.125f, 0,
                                   99, fake(9), size_t(1) << 30, nullptr),
         SQA_ERR_ARG, "bwd varlen split count 99");
}

void layer_and_block() {
  expect(sqa_layer_fwd(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), 16, 1024, 256, 16, 8, 4, 10000.f, 0.25f,
                       1, SQA_BF16, nullptr, 0, nullptr),
         SQA_ERR_WORKSPACE, "layer without workspace");
  expect(sqa_layer_fwd(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), 16, 1024, 250, 16, 8, 4, 10000.f, 0.25f,
                       1, SQA_BF16, fake(6), size_t(1) << 30, nullptr),
         SQA_ERR_SHAPE, "layer D not a multiple of H");
  expect(sqa_layer_fwd(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), 16, 1024, 256, 16, 8, 4, -1.f, 0.25f, 1,
                       SQA_BF16, fake(6), size_t(1) << 30, nullptr),
         SQA_ERR_ARG, "layer rope base");
  expect(sqa_layer_fwd(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), 1, int64_t(1) << 22, 256, 16, 8, 4,
                       10000.f, 0.25f, 1, SQA_BF16, fake(6), size_t(1) << 36, nullptr),
         SQA_ERR_SHAPE, "layer activations of 2^31 bytes");
  expect(sqa_block_fwd(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7), fake(8), fake(9),
                       fake(10), 16, 1024, 256, 16, 8, 4, 770, 10000.f, 0.25f, 1e-6f, 1, SQA_BF16, fake(11),
                       size_t(1) << 30, nullptr),
         SQA_ERR_UNSUPPORTED, "block F not a multiple of 16");
  expect(sqa_block_fwd(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7), fake(8), fake(9),
                       fake(10), 16, 1024, 256, 16, 8, 4, 768, 10000.f, 0.25f, -1.f, 1, SQA_BF16, fake(11),
                       size_t(1) << 30, nullptr),
         SQA_ERR_ARG, "block eps < 0");
  expect(sqa_block_fwd(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7), fake(8), fake(9),
                       fake(10), 1, int64_t(1) << 22, 256, 16, 8, 4, 768, 10000.f, 0.25f, 1e-6f, 1, SQA_BF16,
                       fake(11), size_t(1) << 38, nullptr),
         SQA_ERR_SHAPE, "block activations of 2^31 bytes");
  expect(sqa_block_fwd(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7), fake(8), fake(9),
                       fake(10), 0, 1024, 256, 16, 8, 4, 768, 10000.f, 0.25f, 1e-6f, 1, SQA_BF16, nullptr, 0,
                       nullptr),
         SQA_OK, "block B = 0");
  (void)fake_near;
}

void size_queries() {
  const int64_t ext[] = {INT64_MIN, -1, 0, 1, 1000, int64_t(1) << 31, int64_t(1) << 40, INT64_MAX};
  size_t acc = 0;
  for (int64_t a : ext)
    for (int64_t b : ext) {
      acc += sqa_attn_fwd_split_workspace_bytes(a, 64, SQA_BF16, 2);
      acc += sqa_attn_bwd_workspace_bytes(a, 8, b, 64, SQA_BF16);
      acc += sqa_attn_bwd_varlen_workspace_bytes(a, 8, b, 128, SQA_BF16);
      acc += sqa_attn_bwd_split_workspace_bytes(a, 8, 4, b, 64, SQA_BF16, 3);
      acc += sqa_attn_bwd_varlen_split_workspace_bytes(a, 8, 4, b, 64, SQA_BF16, 3);
      acc += sqa_layer_workspace_bytes(a, b, 256, 16, 8, 4, SQA_BF16);
      acc += sqa_block_workspace_bytes(a, b, 256, 16, 8, 4, 768, SQA_BF16);
      acc += (size_t)sqa_attn_fwd_num_splits(a, 8, 4, b, 64, SQA_BF16, 0, 0);
      acc += (size_t)sqa_attn_fwd_tail_splits(a, 4, 4, b, 64, SQA_BF16, 0);
      acc += sqa_attn_fwd_tail_workspace_bytes(b, 8, 4, a, 64, SQA_BF16, 0);
      acc += (size_t)sqa_attn_bwd_num_splits(a, 8, 4, b, 64, SQA_BF16, 0, 0);
    }
  std::printf("size queries done (%zu)\n", acc);
  for (int s = -1; s < 10; ++s)
    if (sqa_status_str(s) == nullptr) ++g_fail;
  if (sqa_version() < 100) ++g_fail;
}

}  // namespace

int main() {
  attn_forward();
  attn_backward();
  layer_and_block();
  size_queries();
  std::printf("%s: %d failure(s)\n", g_fail ? "FAILED" : "OK", g_fail);
  return g_fail ? 1 : 0;
}
