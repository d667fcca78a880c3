// Host-only driver of libssd's C ABI layer (ssd_api.cpp linked against the
// stand-in launchers), built with AddressSanitizer and
// UndefinedBehaviorSanitizer.  It exercises every entry point's argument
// checks and, for valid calls, checks what reaches the launchers: the shape,
// the dtype flags, the workspace split of ssd_forward and the two-level
// parking flags.  Exits non-zero on the first mismatch; the sanitizers abort
// on the first memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "ssd.h"
#include "stub_launchers.h"

namespace {

int failures = 0;

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

// Host buffers stand in for device memory: the stand-in launchers never
// dereference them, but they are real, 16-byte aligned allocations.
alignas(16) unsigned char arena[1 << 16];
void* P(int k) { return arena + 256 * k; }
void* MIS(int k) { return arena + 256 * k + 4; }

ssd_dims dims(int64_t b = 2, int64_t L = 256, int64_t H = 4, int64_t P_ = 64, int64_t N = 128,
              int64_t G = 2, int64_t T = 64) {
  ssd_dims d{b, L, H, P_, N, G, T};
  return d;
}

ssd_status fwd(const ssd_dims* d, void* ws, size_t wsb, ssd_dtype in = SSD_BF16,
               ssd_dtype yd = SSD_F32, const float* init = nullptr, float* fin = nullptr,
               void* x = P(1)) {
  return ssd_forward(x, (const float*)P(2), (const float*)P(3), P(4), P(5), (const float*)P(6),
                     init, P(7), (float*)P(8), fin, ws, wsb, in, yd, d, nullptr);
}

void test_status_strings() {
  CHECK(std::strcmp(ssd_status_string(SSD_OK), "SSD_OK") == 0);
  CHECK(std::strcmp(ssd_status_string(SSD_ERR_HIP), "SSD_ERR_HIP") == 0);
  CHECK(std::strcmp(ssd_status_string((ssd_status)77), "SSD_ERR_UNKNOWN") == 0);
}

void test_dims_checks() {
  const ssd_dims good = dims();
  CHECK(ssd_forward_workspace_bytes(&good) == 8u * 2 * 4 * 256);
  CHECK(ssd_forward_workspace_bytes(nullptr) == 0);
  struct Case {
    ssd_dims d;
    ssd_status want;
  } cases[] = {
      {dims(0), SSD_ERR_INVALID_ARGUMENT},
      {dims(2, 0), SSD_ERR_INVALID_ARGUMENT},
      {dims(2, 256, -1), SSD_ERR_INVALID_ARGUMENT},
      {dims(2, 256, 4, 64, 128, 3), SSD_ERR_INVALID_ARGUMENT},
      {dims(2, 256, 4, 32), SSD_ERR_UNSUPPORTED},
      {dims(2, 256, 4, 64, 96), SSD_ERR_UNSUPPORTED},
      {dims(2, 256, 4, 64, 128, 2, 32), SSD_ERR_UNSUPPORTED},
      {dims(2, (int64_t)1 << 40), SSD_ERR_INVALID_ARGUMENT},
      {dims(1, (int64_t)1 << 22), SSD_ERR_UNSUPPORTED},
      {dims(INT64_MAX), SSD_ERR_INVALID_ARGUMENT},
      {dims(2, 256, 4, 64, 128, 2, INT64_MIN), SSD_ERR_INVALID_ARGUMENT},
      // block counts past 32 bits, with products that would overflow 64
      {dims((int64_t)1 << 30, 1, (int64_t)1 << 30, 64, 128, 1, 64), SSD_ERR_INVALID_ARGUMENT},
      {dims(INT32_MAX, 1, INT32_MAX, 64, 128, 1, 64), SSD_ERR_INVALID_ARGUMENT},
  };
  for (const Case& c : cases) {
    stub::reset();
    CHECK(fwd(&c.d, P(20), 1 << 20) == c.want);
    CHECK(stub::ncalls == 0);
    CHECK(ssd_forward_workspace_bytes(&c.d) == 0);
  }
}

void test_forward() {
  const ssd_dims d = dims(2, 300, 4, 64, 128, 2, 128);
  const size_t need = ssd_forward_workspace_bytes(&d);
  CHECK(need == 8u * 2 * 4 * 300);
  // rejected before any launch
  stub::reset();
  CHECK(fwd(&d, P(20), need - 1) == SSD_ERR_WORKSPACE);
  CHECK(fwd(&d, nullptr, need) == SSD_ERR_WORKSPACE);
  CHECK(fwd(&d, MIS(20), need) == SSD_ERR_WORKSPACE);
  CHECK(fwd(&d, P(20), need, (ssd_dtype)2) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(fwd(&d, P(20), need, SSD_BF16, (ssd_dtype)-1) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(fwd(&d, P(20), need, SSD_BF16, SSD_F32, nullptr, nullptr, MIS(1)) ==
        SSD_ERR_INVALID_ARGUMENT);
  CHECK(fwd(&d, P(20), need, SSD_BF16, SSD_F32, (const float*)MIS(9)) ==
        SSD_ERR_INVALID_ARGUMENT);
  CHECK(fwd(nullptr, P(20), need) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(stub::ncalls == 0);
  // a valid call: stage 1, then stages 2 and 3, g and dt_t split from the
  // workspace, the dtype flags passed through
  float* ws = (float*)P(20);
  CHECK(fwd(&d, ws, need, SSD_BF16, SSD_BF16, (const float*)P(9), (float*)P(9)) == SSD_OK);
  CHECK(stub::ncalls == 2);
  CHECK(std::strcmp(stub::calls[0].name, "chunk_cumsum") == 0);
  CHECK(std::strcmp(stub::calls[1].name, "state_and_out") == 0);
  CHECK(stub::calls[0].p[1] == ws && stub::calls[0].p[2] == ws + 2 * 4 * 300);
  CHECK(stub::calls[1].p[0] == ws + 2 * 4 * 300 && stub::calls[1].p[1] == ws &&
        stub::calls[1].p[2] == P(8));
  CHECK(stub::calls[1].flag[0] && stub::calls[1].flag[1]);
  CHECK(stub::calls[1].shape.seqlen == 300 && stub::calls[1].shape.chunk == 128 &&
        stub::calls[1].shape.nchunks() == 3 && stub::calls[1].shape.ngroups == 2);
  // a failing launch stops the sequence and maps to SSD_ERR_HIP
  stub::reset();
  stub::fail_with = 98;
  CHECK(fwd(&d, ws, need) == SSD_ERR_HIP);
  CHECK(stub::ncalls == 1);
  stub::reset();
}

void test_forward_noalloc() {
  auto call = [](const ssd_dims* d, ssd_dtype in = SSD_BF16) {
    return ssd_forward_noalloc(P(1), (const float*)P(2), (const float*)P(3), P(4), P(5),
                               (const float*)P(6), nullptr, P(7), (float*)P(8), nullptr, in,
                               SSD_F32, d, nullptr);
  };
  stub::reset();
  const ssd_dims d = dims(2, 300, 4, 64, 128, 2, 128);
  CHECK(call(&d) == SSD_OK);
  CHECK(stub::ncalls == 1 && std::strcmp(stub::calls[0].name, "forward_noalloc") == 0);
  CHECK(stub::calls[0].shape.seqlen == 300 && stub::calls[0].flag[0]);
  // g and dt_t must fit the per-GPU scratch array: 8 * b * H * L bytes
  const int64_t fit = (int64_t)(SSD_NOALLOC_SCRATCH_BYTES / 8 / 64);   // b * L with H = 64
  const ssd_dims at = dims(1, fit, 64, 64, 64, 1, 64);
  const ssd_dims over = dims(1, fit + 1, 64, 64, 64, 1, 64);
  CHECK(ssd_forward_workspace_bytes(&at) == SSD_NOALLOC_SCRATCH_BYTES);
  CHECK(call(&at) == SSD_OK);
  CHECK(call(&over) == SSD_ERR_WORKSPACE);
  CHECK(call(&d, (ssd_dtype)3) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(call(nullptr) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(stub::ncalls == 2);
  stub::reset();
}

void test_stage_entry_points() {
  const ssd_dims d = dims();
  stub::reset();
  // stage 1 reads only batch, seqlen, nheads and chunk size
  ssd_dims odd = dims(2, 256, 4, 7, 3, 3, 64);
  CHECK(ssd_chunk_cumsum((const float*)P(1), (const float*)P(2), (float*)P(3), (float*)P(4),
                         &odd, nullptr) == SSD_OK);
  CHECK(stub::ncalls == 1 && stub::calls[0].shape.nheads == 4);
  CHECK(ssd_chunk_cumsum((const float*)P(1), (const float*)P(2), (float*)MIS(3), (float*)P(4),
                         &d, nullptr) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(ssd_fwd_pass_state(P(1), P(2), (const float*)P(3), (const float*)P(4), nullptr,
                           (float*)P(5), nullptr, SSD_F32, &d, nullptr) == SSD_OK);
  CHECK(!stub::calls[1].flag[0]);
  CHECK(ssd_fwd_pass_state(P(1), P(2), (const float*)P(3), (const float*)P(4), nullptr,
                           nullptr, nullptr, SSD_F32, &d, nullptr) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(ssd_compute_out(P(1), P(2), P(3), (const float*)P(4), (const float*)P(5),
                        (const float*)P(6), (const float*)P(7), P(8), SSD_F32, SSD_BF16, &d,
                        nullptr) == SSD_OK);
  CHECK(!stub::calls[2].flag[0] && stub::calls[2].flag[1]);
  CHECK(ssd_compute_out(P(1), P(2), P(3), (const float*)P(4), (const float*)P(5),
                        (const float*)P(6), nullptr, P(8), SSD_F32, SSD_BF16, &d,
                        nullptr) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(stub::ncalls == 3);
  // stages 2 and 3 in one call: optional init/final, dtype flags through
  CHECK(ssd_state_and_out(P(1), P(2), P(3), (const float*)P(4), (const float*)P(5),
                          (const float*)P(6), nullptr, P(7), (float*)P(8), nullptr, SSD_F32,
                          SSD_BF16, &d, nullptr) == SSD_OK);
  CHECK(stub::ncalls == 4 && std::strcmp(stub::calls[3].name, "state_and_out") == 0);
  CHECK(stub::calls[3].p[0] == P(4) && stub::calls[3].p[1] == P(5) &&
        stub::calls[3].p[2] == P(8));
  CHECK(!stub::calls[3].flag[0] && stub::calls[3].flag[1]);
  CHECK(ssd_state_and_out(P(1), P(2), P(3), (const float*)P(4), (const float*)P(5),
                          (const float*)P(6), (const float*)MIS(9), P(7), (float*)P(8),
                          nullptr, SSD_F32, SSD_F32, &d,
                          nullptr) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(ssd_state_and_out(P(1), P(2), P(3), (const float*)P(4), nullptr,
                          (const float*)P(6), nullptr, P(7), (float*)P(8), nullptr, SSD_F32,
                          SSD_F32, &d, nullptr) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(ssd_state_and_out(P(1), P(2), P(3), (const float*)P(4), (const float*)P(5),
                          (const float*)P(6), nullptr, P(7), (float*)P(8), nullptr,
                          (ssd_dtype)7, SSD_F32, &d, nullptr) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(stub::ncalls == 4);
}

void test_two_level() {
  const ssd_dims d = dims();
  stub::reset();
  // the public two-call form never parks
  CHECK(ssd_chunk_state(P(1), P(2), (const float*)P(3), (const float*)P(4), (float*)P(5),
                        (float*)P(6), SSD_BF16, &d, nullptr) == SSD_OK);
  CHECK(stub::ncalls == 1 && !stub::calls[0].flag[1]);
  // init may not overlap final in the two-call form: whole, partial, or
  // starting inside it (a state here is 2 * 4 * 64 * 128 floats)
  const size_t sb = 4u * 2 * 4 * 64 * 128;
  unsigned char* big = (unsigned char*)std::aligned_alloc(16, 3 * sb);
  CHECK(ssd_state_passing((const float*)P(4), (const float*)big, (float*)P(5),
                          (float*)(big + 2 * sb), &d, nullptr) == SSD_OK);
  CHECK(stub::ncalls == 2 && !stub::calls[1].flag[0]);
  CHECK(ssd_state_passing((const float*)P(4), (const float*)big, (float*)P(5), (float*)big, &d,
                          nullptr) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(ssd_state_passing((const float*)P(4), (const float*)(big + sb - 16), (float*)P(5),
                          (float*)big, &d, nullptr) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(ssd_state_passing((const float*)P(4), (const float*)big, (float*)P(5),
                          (float*)(big + sb - 16), &d, nullptr) == SSD_ERR_INVALID_ARGUMENT);
  // adjacent, not overlapping
  CHECK(ssd_state_passing((const float*)P(4), (const float*)big, (float*)P(5),
                          (float*)(big + sb), &d, nullptr) == SSD_OK);
  std::free(big);
  CHECK(stub::ncalls == 3);
  // the one-call stage 2 accepts init == final
  CHECK(ssd_fwd_pass_state(P(1), P(2), (const float*)P(3), (const float*)P(4),
                           (const float*)P(9), (float*)P(5), (float*)P(9), SSD_BF16, &d,
                           nullptr) == SSD_OK);
  stub::reset();
}

void test_side_entry_points() {
  const ssd_dims d = dims();
  stub::reset();
  CHECK(ssd_decode_step(P(1), (const float*)P(2), (const float*)P(3), P(4), P(5),
                        (const float*)P(6), (float*)P(7), P(8), SSD_BF16, SSD_F32, &d,
                        nullptr) == SSD_OK);
  CHECK(stub::calls[0].shape.seqlen == 1);
  CHECK(ssd_decode_step(P(1), (const float*)P(2), (const float*)P(3), P(4), P(5),
                        (const float*)P(6), (float*)P(7), P(8), (ssd_dtype)5, SSD_F32, &d,
                        nullptr) == SSD_ERR_INVALID_ARGUMENT);
  CHECK(ssd_causal_conv1d(P(1), (const float*)P(2), nullptr, P(3), 2, 8, 64, 4, SSD_BF16,
                          SSD_F32, nullptr) == SSD_OK);
  CHECK(ssd_causal_conv1d(P(1), (const float*)P(2), nullptr, P(3), 2, 8, 64, 5, SSD_BF16,
                          SSD_F32, nullptr) == SSD_ERR_UNSUPPORTED);
  CHECK(ssd_causal_conv1d(P(1), (const float*)P(2), nullptr, P(3), (int64_t)1 << 30, 1 << 12,
                          1 << 12, 4, SSD_BF16, SSD_F32, nullptr) == SSD_ERR_UNSUPPORTED);
  ssd_gdn_dims gd{2, 256, 4, 128, 128, 64};
  CHECK(ssd_gdn_chunk_fwd_h(P(1), P(2), P(3), (const float*)P(4), nullptr, (float*)P(5), P(6),
                            nullptr, SSD_BF16, SSD_BF16, &gd, nullptr) == SSD_OK);
  CHECK(ssd_gdn_chunk_fwd_o(P(1), P(2), P(3), (const float*)P(4), (const float*)P(5), P(6),
                            1.0f, SSD_BF16, SSD_BF16, SSD_F32, &gd, nullptr) == SSD_OK);
  ssd_gdn_dims huge{INT32_MAX, 1, INT32_MAX, 128, 128, 64};
  CHECK(ssd_gdn_chunk_fwd_h(P(1), P(2), P(3), (const float*)P(4), nullptr, (float*)P(5), P(6),
                            nullptr, SSD_BF16, SSD_BF16, &huge, nullptr) ==
        SSD_ERR_INVALID_ARGUMENT);
  gd.dk = 96;
  CHECK(ssd_gdn_chunk_fwd_h(P(1), P(2), P(3), (const float*)P(4), nullptr, (float*)P(5), P(6),
                            nullptr, SSD_BF16, SSD_BF16, &gd, nullptr) == SSD_ERR_UNSUPPORTED);
  CHECK(stub::ncalls == 4);
  stub::reset();
}

}  // namespace

int main() {
  test_status_strings();
  test_dims_checks();
  test_forward();
  test_forward_noalloc();
  test_stage_entry_points();
  test_two_level();
  test_side_entry_points();
  if (failures) {
    std::fprintf(stderr, "abi_driver: %d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi_driver: all checks passed\n");
  return 0;
}
