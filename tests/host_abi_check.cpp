// Host-side checks of libmqa's C ABI, built and run under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only) by tests/test_host_sanitizers.py. Every call
// below is rejected by the argument checks, or is a size query, before any HIP work is
// enqueued, so no GPU is needed. Fake device pointers are never dereferenced.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "mqa.h"
#include "mqa_probe.h"

namespace {

int failures = 0, checks = 0;

void expect(int got, int want, const char* what) {
  ++checks;
  if (got != want) {
    ++failures;
    std::printf("FAIL %s: status %d, want %d\n", what, got, want);
  }
}

void expect_true(bool ok, const char* what) {
  ++checks;
  if (!ok) {
    ++failures;
    std::printf("FAIL %s\n", what);
  }
}

template <typename T>
T* fake(uintptr_t addr) {
  return reinterpret_cast<T*>(addr);
}

mqa_shape good_shape() {
  mqa_shape s;
  std::memset(&s, 0, sizeof(s));
  s.batch = 2;
  s.next_n = 2;
  s.heads = 64;
  s.head_dim = 128;
  s.block_size = 1;
  s.block_table_stride = 100;
  s.num_blocks = 1000;
  return s;
}

int logits(const mqa_shape* s, int32_t L, uintptr_t q = 0x10000, uintptr_t kv = 0x10000, uintptr_t w = 0x10000,
           uintptr_t ctx = 0x10000, uintptr_t bt = 0x10000, uintptr_t out = 0x10000) {
  return mqa_paged_logits(fake<const uint8_t>(q), fake<const uint8_t>(kv), fake<const float>(w),
                          fake<const int32_t>(ctx), fake<const int32_t>(bt), L, fake<float>(out), s, nullptr);
}

int topk(const mqa_shape* s, int32_t L, int32_t k = 2048, uintptr_t ws = 0, size_t ws_bytes = 0,
         uintptr_t lg = 0x10000, uintptr_t ctx = 0x10000, uintptr_t idx = 0x10000) {
  return mqa_topk(fake<const float>(lg), fake<const int32_t>(ctx), L, k, fake<int32_t>(idx), s, fake<void>(ws),
                  ws_bytes, nullptr);
}

int topk_noalloc(const mqa_shape* s, int32_t L, int32_t k = 2048, uintptr_t lg = 0x10000, uintptr_t ctx = 0x10000,
                 uintptr_t idx = 0x10000) {
  return mqa_topk_noalloc(fake<const float>(lg), fake<const int32_t>(ctx), L, k, fake<int32_t>(idx), s, nullptr);
}

void check_shapes() {
  struct Case {
    const char* what;
    void (*edit)(mqa_shape&);
    int32_t L;
    int want;
  };
  const Case cases[] = {
      {"batch -1", [](mqa_shape& s) { s.batch = -1; }, 100, MQA_ERR_SHAPE},
      {"next_n 0", [](mqa_shape& s) { s.next_n = 0; }, 100, MQA_ERR_SHAPE},
      {"heads 0", [](mqa_shape& s) { s.heads = 0; }, 100, MQA_ERR_SHAPE},
      {"num_blocks 0", [](mqa_shape& s) { s.num_blocks = 0; }, 100, MQA_ERR_SHAPE},
      {"stride 0", [](mqa_shape& s) { s.block_table_stride = 0; }, 100, MQA_ERR_SHAPE},
      {"L 0", [](mqa_shape&) {}, 0, MQA_ERR_SHAPE},
      {"head_dim 64", [](mqa_shape& s) { s.head_dim = 64; }, 100, MQA_ERR_UNSUPPORTED},
      {"block_size 0", [](mqa_shape& s) { s.block_size = 0; }, 100, MQA_ERR_SHAPE},
      {"block_size 3", [](mqa_shape& s) { s.block_size = 3; }, 100, MQA_ERR_UNSUPPORTED},
      {"block_size 48", [](mqa_shape& s) { s.block_size = 48; }, 100, MQA_ERR_UNSUPPORTED},
      {"block_size 2^17", [](mqa_shape& s) { s.block_size = 1 << 17; }, 100, MQA_ERR_UNSUPPORTED},
      {"W*S >= 2^31", [](mqa_shape& s) { s.block_size = 64; s.block_table_stride = 1 << 25; }, 100, MQA_ERR_UNSUPPORTED},
      {"blocks*S >= 2^31", [](mqa_shape& s) { s.block_size = 64; s.num_blocks = 1 << 25; }, 100, MQA_ERR_UNSUPPORTED},
      {"heads 24", [](mqa_shape& s) { s.heads = 24; }, 100, MQA_ERR_UNSUPPORTED},
      {"heads 144", [](mqa_shape& s) { s.heads = 144; }, 100, MQA_ERR_UNSUPPORTED},
      {"next_n 5", [](mqa_shape& s) { s.next_n = 5; }, 100, MQA_ERR_UNSUPPORTED},
      {"L 2^30 + 1", [](mqa_shape&) {}, (1 << 30) + 1, MQA_ERR_UNSUPPORTED},
      {"batch * next_n overflow", [](mqa_shape& s) { s.batch = 1 << 30; s.next_n = 4; }, 100, MQA_ERR_SHAPE},
  };
  for (const Case& c : cases) {
    mqa_shape s = good_shape();
    c.edit(s);
    expect(logits(&s, c.L), c.want, c.what);
    expect(topk(&s, c.L), c.want, c.what);
    expect(topk_noalloc(&s, c.L), c.want, c.what);
  }
}

void check_pointers() {
  mqa_shape s = good_shape();
  expect(logits(nullptr, 100), MQA_ERR_NULL, "logits shape NULL");
  expect(topk(nullptr, 100), MQA_ERR_NULL, "topk shape NULL");
  expect(topk_noalloc(nullptr, 100), MQA_ERR_NULL, "topk_noalloc shape NULL");
  for (int i = 0; i < 6; ++i) {  // one pointer NULL, then one misaligned
    uintptr_t p[6] = {0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000};
    p[i] = 0;
    expect(logits(&s, 100, p[0], p[1], p[2], p[3], p[4], p[5]), MQA_ERR_NULL, "logits pointer NULL");
    p[i] = 0x10002;
    expect(logits(&s, 100, p[0], p[1], p[2], p[3], p[4], p[5]), MQA_ERR_UNSUPPORTED, "logits pointer misaligned");
  }
  for (int i = 0; i < 3; ++i) {
    uintptr_t p[3] = {0x10000, 0x10000, 0x10000};
    p[i] = 0;
    expect(topk(&s, 100, 2048, 0, 0, p[0], p[1], p[2]), MQA_ERR_NULL, "topk pointer NULL");
    expect(topk_noalloc(&s, 100, 2048, p[0], p[1], p[2]), MQA_ERR_NULL, "topk_noalloc pointer NULL");
    p[i] = 0x10002;
    expect(topk(&s, 100, 2048, 0, 0, p[0], p[1], p[2]), MQA_ERR_UNSUPPORTED, "topk pointer misaligned");
    expect(topk_noalloc(&s, 100, 2048, p[0], p[1], p[2]), MQA_ERR_UNSUPPORTED, "topk_noalloc pointer misaligned");
  }
  expect(logits(&s, 100, 0x10004), MQA_ERR_UNSUPPORTED, "q not 16-byte aligned");
  expect(logits(&s, 100, 0x10000, 0x10000, 0x10004), MQA_ERR_UNSUPPORTED, "weights not 16-byte aligned");
  mqa_shape empty = good_shape();
  empty.batch = 0;
  expect(logits(&empty, 100, 0, 0, 0, 0, 0, 0), MQA_OK, "empty batch logits with NULL data");
  expect(topk(&empty, 100, 2048, 0, 0, 0, 0, 0), MQA_OK, "empty batch topk with NULL data");
  expect(topk_noalloc(&empty, 100, 2048, 0, 0, 0), MQA_OK, "empty batch topk_noalloc with NULL data");
}

void check_limits() {
  mqa_shape s = good_shape();
  s.batch = 8193;
  expect(logits(&s, 100), MQA_ERR_UNSUPPORTED, "logits batch 8193");
  s = good_shape();
  s.batch = 8192;
  s.next_n = 4;
  expect(logits(&s, 1 << 30), MQA_ERR_UNSUPPORTED, "logits work count above 2^31");
  s.batch = 1024;
  expect(logits(&s, 1 << 25), MQA_ERR_UNSUPPORTED, "logits work count 4096 * (2^19 + 1)");
  s = good_shape();
  expect(topk(&s, 100, 0), MQA_ERR_SHAPE, "k 0");
  expect(topk(&s, 100, 2049), MQA_ERR_UNSUPPORTED, "k 2049");
}

void check_workspace() {
  mqa_shape s = good_shape();
  s.block_table_stride = 40000;
  const size_t need = mqa_topk_workspace_bytes(&s, 40000, 2048);
  expect_true(need > 0, "workspace needed above 32768");
  expect_true(mqa_topk_workspace_bytes(&s, 32768, 2048) == 0, "no workspace up to 32768");
  expect_true(mqa_topk_workspace_bytes(&s, 32769, 2048) > 0, "workspace above 32768");
  expect_true(mqa_topk_workspace_bytes(&s, 100, 0) == 0, "workspace size for k 0");
  expect_true(mqa_topk_workspace_bytes(nullptr, 40000, 2048) == 0, "workspace size of NULL shape");
  expect(topk(&s, 40000), MQA_ERR_WORKSPACE, "workspace missing");
  expect(topk(&s, 40000, 2048, 0x10000, need - 1), MQA_ERR_WORKSPACE, "workspace short");
  expect(topk(&s, 40000, 2048, 0x10008, need), MQA_ERR_WORKSPACE, "workspace not 16-byte aligned");
  mqa_shape big = good_shape();
  big.batch = 1024;
  big.next_n = 1;
  big.block_table_stride = 202752;
  expect_true(mqa_topk_workspace_bytes(&big, 202752, 2048) > (size_t(64) << 20), "big shape needs > 64 MiB");
  expect(topk_noalloc(&big, 202752), MQA_ERR_SCRATCH, "noalloc beyond the static scratch");
  mqa_shape ok = big;
  ok.batch = 128;
  ok.next_n = 4;
  const size_t ok_need = mqa_topk_workspace_bytes(&ok, 202752, 2048);
  expect_true(ok_need > 0 && ok_need <= (size_t(64) << 20), "512 long rows fit the static scratch");
  expect(topk_noalloc(&ok, 202752, 2048, 0, 0, 0), MQA_ERR_NULL, "noalloc within the scratch, NULL data");
}

void check_other_entry_points() {
  // K-cache write
  expect(mqa_indexer_k_write(fake<void>(0x10000), MQA_DTYPE_BF16, -1, fake<const int64_t>(0x10000),
                             fake<uint8_t>(0x10000), 100, nullptr),
         MQA_ERR_SHAPE, "kwrite negative tokens");
  expect(mqa_indexer_k_write(fake<void>(0x10000), 7, 4, fake<const int64_t>(0x10000), fake<uint8_t>(0x10000), 100,
                             nullptr),
         MQA_ERR_UNSUPPORTED, "kwrite bad dtype");
  expect(mqa_indexer_k_write(nullptr, MQA_DTYPE_BF16, 4, fake<const int64_t>(0x10000), fake<uint8_t>(0x10000), 100,
                             nullptr),
         MQA_ERR_NULL, "kwrite NULL keys");
  expect(mqa_indexer_k_write(fake<void>(0x10008), MQA_DTYPE_BF16, 4, fake<const int64_t>(0x10000),
                             fake<uint8_t>(0x10000), 100, nullptr),
         MQA_ERR_UNSUPPORTED, "kwrite keys not 16-byte aligned");
  expect(mqa_indexer_k_write(nullptr, MQA_DTYPE_BF16, 0, nullptr, nullptr, 100, nullptr), MQA_OK, "kwrite no tokens");
  // non-paged logits
  expect(mqa_logits(fake<const uint8_t>(0x10000), fake<const uint8_t>(0x10000), fake<const float>(0x10000),
                    fake<const float>(0x10000), fake<const int32_t>(0x10000), fake<const int32_t>(0x10000),
                    fake<float>(0x10000), 50, 4, 100, 32, nullptr),
         MQA_ERR_SHAPE, "prefill stride below n");
  expect(mqa_logits(fake<const uint8_t>(0x10000), fake<const uint8_t>(0x10000), fake<const float>(0x10000),
                    fake<const float>(0x10000), fake<const int32_t>(0x10000), fake<const int32_t>(0x10000),
                    fake<float>(0x10000), 100, 4, 100, 80, nullptr),
         MQA_ERR_UNSUPPORTED, "prefill heads 80");
  expect(mqa_logits(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 100, 0, 100, 32, nullptr), MQA_OK,
         "prefill no rows");
  struct PrefillCase {
    const char* what;
    int32_t m, n, heads;
    int64_t stride;
    int bad_ptr;  // index of a pointer replaced by bad_val, or -1
    uintptr_t bad_val;
    int want;
  };
  const PrefillCase prefill_cases[] = {
      {"prefill m -1", -1, 64, 32, 64, -1, 0, MQA_ERR_SHAPE},
      {"prefill n 0", 4, 0, 32, 64, -1, 0, MQA_ERR_SHAPE},
      {"prefill heads 0", 4, 64, 0, 64, -1, 0, MQA_ERR_SHAPE},
      {"prefill heads 24", 4, 64, 24, 64, -1, 0, MQA_ERR_UNSUPPORTED},
      {"prefill n 2^29 + 1", 4, (1 << 29) + 1, 32, (1 << 29) + 1, -1, 0, MQA_ERR_UNSUPPORTED},
      {"prefill q NULL", 4, 64, 32, 64, 0, 0, MQA_ERR_NULL},
      {"prefill out NULL", 4, 64, 32, 64, 6, 0, MQA_ERR_NULL},
      {"prefill q misaligned", 4, 64, 32, 64, 0, 0x10008, MQA_ERR_UNSUPPORTED},
      {"prefill k misaligned", 4, 64, 32, 64, 1, 0x10004, MQA_ERR_UNSUPPORTED},
      {"prefill weights misaligned", 4, 64, 32, 64, 3, 0x10004, MQA_ERR_UNSUPPORTED},
  };
  for (const PrefillCase& c : prefill_cases) {
    uintptr_t p[7] = {0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000};
    if (c.bad_ptr >= 0) p[c.bad_ptr] = c.bad_val;
    expect(mqa_logits(fake<const uint8_t>(p[0]), fake<const uint8_t>(p[1]), fake<const float>(p[2]),
                      fake<const float>(p[3]), fake<const int32_t>(p[4]), fake<const int32_t>(p[5]),
                      fake<float>(p[6]), c.stride, c.m, c.n, c.heads, nullptr),
           c.want, c.what);
  }
  // sparse MLA decode
  mqa_mla_shape m;
  std::memset(&m, 0, sizeof(m));
  m.batch = 2;
  m.next_n = 2;
  m.heads = 16;
  m.head_dim = 576;
  m.v_dim = 512;
  m.block_size = 1;
  m.block_table_stride = 100;
  m.topk = 64;
  m.num_blocks = 1000;
  auto mla = [](const mqa_mla_shape* sh, const uintptr_t* p, uintptr_t lse = 0, uintptr_t ws = 0,
                size_t ws_bytes = 0) {
    return mqa_sparse_mla_decode(fake<const uint8_t>(p[0]), 1.0f, fake<const uint8_t>(p[1]), 1.0f,
                                 fake<const int32_t>(p[2]), fake<const int32_t>(p[3]), 0.07f, fake<float>(p[4]),
                                 fake<float>(lse), sh, fake<void>(ws), ws_bytes, nullptr);
  };
  const uintptr_t good[5] = {0x10000, 0x10000, 0x10000, 0x10000, 0x10000};
  struct MlaCase {
    const char* what;
    void (*edit)(mqa_mla_shape&);
    int want;
  };
  const MlaCase mla_cases[] = {
      {"mla batch -1", [](mqa_mla_shape& x) { x.batch = -1; }, MQA_ERR_SHAPE},
      {"mla next_n 0", [](mqa_mla_shape& x) { x.next_n = 0; }, MQA_ERR_SHAPE},
      {"mla topk 0", [](mqa_mla_shape& x) { x.topk = 0; }, MQA_ERR_SHAPE},
      {"mla block_size 0", [](mqa_mla_shape& x) { x.block_size = 0; }, MQA_ERR_SHAPE},
      {"mla stride 0", [](mqa_mla_shape& x) { x.block_table_stride = 0; }, MQA_ERR_SHAPE},
      {"mla num_blocks 0", [](mqa_mla_shape& x) { x.num_blocks = 0; }, MQA_ERR_SHAPE},
      {"mla heads 32", [](mqa_mla_shape& x) { x.heads = 32; }, MQA_ERR_UNSUPPORTED},
      {"mla head_dim 512", [](mqa_mla_shape& x) { x.head_dim = 512; }, MQA_ERR_UNSUPPORTED},
      {"mla v_dim 576", [](mqa_mla_shape& x) { x.v_dim = 576; }, MQA_ERR_UNSUPPORTED},
      {"mla block_size 3", [](mqa_mla_shape& x) { x.block_size = 3; }, MQA_ERR_UNSUPPORTED},
      {"mla block_size 2^17", [](mqa_mla_shape& x) { x.block_size = 1 << 17; }, MQA_ERR_UNSUPPORTED},
      {"mla W*S >= 2^31", [](mqa_mla_shape& x) { x.block_size = 64; x.block_table_stride = 1 << 25; },
       MQA_ERR_UNSUPPORTED},
      {"mla blocks*S >= 2^31", [](mqa_mla_shape& x) { x.block_size = 64; x.num_blocks = 1 << 25; },
       MQA_ERR_UNSUPPORTED},
      {"mla rows 65536", [](mqa_mla_shape& x) { x.batch = 65536; x.next_n = 1; }, MQA_ERR_UNSUPPORTED},
      {"mla topk 2^20 + 1", [](mqa_mla_shape& x) { x.topk = (1 << 20) + 1; }, MQA_ERR_UNSUPPORTED},
  };
  for (const MlaCase& c : mla_cases) {
    mqa_mla_shape x = m;
    c.edit(x);
    expect(mla(&x, good), c.want, c.what);
    expect_true(mqa_sparse_mla_workspace_bytes(&x) == 0, "mla workspace of a rejected shape");
  }
  expect(mla(nullptr, good), MQA_ERR_NULL, "mla shape NULL");
  for (int i = 0; i < 5; ++i) {
    uintptr_t p[5] = {0x10000, 0x10000, 0x10000, 0x10000, 0x10000};
    p[i] = 0;
    expect(mla(&m, p), MQA_ERR_NULL, "mla pointer NULL");
    p[i] = (i == 2 || i == 3) ? 0x10002 : 0x10008;  // indices and tables need 4 bytes, the rest 16
    expect(mla(&m, p), MQA_ERR_UNSUPPORTED, "mla pointer misaligned");
  }
  expect(mla(&m, good, 0x10002), MQA_ERR_UNSUPPORTED, "mla lse misaligned");
  mqa_mla_shape none = m;
  none.batch = 0;
  const uintptr_t nulls[5] = {0, 0, 0, 0, 0};
  expect(mla(&none, nulls), MQA_OK, "mla no rows");
  mqa_mla_shape big_mla = m;
  big_mla.batch = 64;
  big_mla.next_n = 1;
  big_mla.topk = 2048;
  const size_t mla_need = mqa_sparse_mla_workspace_bytes(&big_mla);
  expect_true(mla_need > 0, "mla workspace needed");
  expect(mla(&big_mla, good), MQA_ERR_WORKSPACE, "mla workspace missing");
  expect(mla(&big_mla, good, 0, 0x10000, mla_need - 1), MQA_ERR_WORKSPACE, "mla workspace short");
  // measurement probe
  expect(mqa_probe_gather(fake<const uint8_t>(0x10000), 10, fake<const int32_t>(0x10000), -1, 2, 2,
                          fake<int32_t>(0x10000), 1 << 20, nullptr),
         2, "probe negative n");
  expect(mqa_probe_gather(fake<const uint8_t>(0x10000), 10, fake<const int32_t>(0x10000), 5, 2, 3,
                          fake<int32_t>(0x10000), 1 << 20, nullptr),
         3, "probe stages 3");
  expect(mqa_probe_gather(fake<const uint8_t>(0x10000), 10, fake<const int32_t>(0x10000), 5, 9, 2,
                          fake<int32_t>(0x10000), 1 << 20, nullptr),
         3, "probe groups_per_cu 9");
  expect(mqa_probe_gather(nullptr, 10, fake<const int32_t>(0x10000), 5, 2, 2, fake<int32_t>(0x10000), 1 << 20,
                          nullptr),
         1, "probe cache NULL");
  expect(mqa_probe_gather(fake<const uint8_t>(0x10000), 10, fake<const int32_t>(0x10000), 0, 2, 2,
                          fake<int32_t>(0x10000), 0, nullptr),
         0, "probe nothing to read");
  expect_true(mqa_probe_gather_sink_words(2) > 0, "probe sink size");
  expect(mqa_probe_gather_lds(fake<const uint8_t>(0x10000), 10, fake<const int32_t>(0x10000), 5, 2, 4,
                              fake<int32_t>(0x10000), 1 << 20, nullptr),
         3, "lds probe stages 4");
  expect(mqa_probe_gather_lds(fake<const uint8_t>(0x10004), 10, fake<const int32_t>(0x10000), 5, 2, 3,
                              fake<int32_t>(0x10000), 1 << 20, nullptr),
         3, "lds probe cache not 16-byte aligned");
  expect(mqa_probe_gather_lds(nullptr, 10, fake<const int32_t>(0x10000), 0, 2, 2, fake<int32_t>(0x10000), 0,
                              nullptr),
         0, "lds probe nothing to read");
  // status strings
  for (int st = -1; st <= 8; ++st) expect_true(mqa_status_string(st) != nullptr, "status string");
  expect_true(std::strcmp(mqa_status_string(MQA_OK), "ok") == 0, "status string of MQA_OK");
}

}  // namespace

int main() {
  check_shapes();
  check_pointers();
  check_limits();
  check_workspace();
  check_other_entry_points();
  std::printf("%s: %d checks, %d failed\n", failures ? "FAILED" : "ok", checks, failures);
  return failures ? 1 : 0;
}
