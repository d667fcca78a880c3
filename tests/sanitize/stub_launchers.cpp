// Stand-ins for libssd's kernel launchers (declared in ssd_launch.h), for a
// host-only build of the C ABI layer (ssd_api.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer.  Each records its call and returns the
// status the driver asks for; none touches the pointers it receives.
#include "stub_launchers.h"

namespace stub {
Call calls[kMaxCalls];
int ncalls = 0;
int fail_with = 0;

static int record(const char* name, const ssd::Shape* s, const void* a, const void* b,
                  const void* c, bool f0, bool f1) {
  if (ncalls < kMaxCalls) {
    Call& k = calls[ncalls];
    k.name = name;
    k.has_shape = s != nullptr;
    if (s) k.shape = *s;
    k.p[0] = a;
    k.p[1] = b;
    k.p[2] = c;
    k.flag[0] = f0;
    k.flag[1] = f1;
  }
  ++ncalls;
  return fail_with;
}
void reset() {
  ncalls = 0;
  fail_with = 0;
}
}  // namespace stub

namespace ssd {

int launch_chunk_cumsum(const float* dt, const float*, float* g, float* dt_t, const Shape& s,
                        void*) {
  return stub::record("chunk_cumsum", &s, dt, g, dt_t, false, false);
}
int launch_fwd_pass_state(const void* x, const void*, const float* dt_t, const float* g,
                          const float*, float* states, float*, bool bf16_in, const Shape& s,
                          void*) {
  (void)dt_t;
  return stub::record("fwd_pass_state", &s, x, g, states, bf16_in, false);
}
int launch_compute_out(const void* x, const void*, const void*, const float* dt_t,
                       const float* g, const float*, const float*, void* y, bool bf16_in,
                       bool bf16_out, const Shape& s, void*) {
  (void)x;
  return stub::record("compute_out", &s, dt_t, g, y, bf16_in, bf16_out);
}
int launch_state_and_out(const void*, const void*, const void*, const float* dt_t,
                         const float* g, const float*, const float*, float* states, float*,
                         void*, bool bf16_in, bool bf16_out, const Shape& s, void*) {
  return stub::record("state_and_out", &s, dt_t, g, states, bf16_in, bf16_out);
}
int launch_chunk_state(const void* x, const void*, const float*, const float*, float* states,
                       float* fin, bool bf16_in, bool park, const Shape& s, void*) {
  return stub::record("chunk_state", &s, x, states, fin, bf16_in, park);
}
int launch_state_passing(const float* g, const float* init, float* states, float*, bool parked,
                         const Shape& s, void*) {
  return stub::record("state_passing", &s, g, init, states, parked, false);
}
int launch_forward_noalloc(const void* x, const float*, const float*, const void*, const void*,
                           const float*, const float*, void* y, float* states, float*,
                           bool bf16_in, bool bf16_out, const Shape& s, void*) {
  return stub::record("forward_noalloc", &s, x, y, states, bf16_in, bf16_out);
}
int launch_decode_step(const void* x, const float*, const float*, const void*, const void*,
                       const float*, float* state, void* y, bool bf16_in, bool bf16_out,
                       const Shape& s, void*) {
  return stub::record("decode_step", &s, x, state, y, bf16_in, bf16_out);
}
int launch_gdn_fwd_h(const void* k, const void*, const void*, const float*, const float*,
                     float* hout, void* vnew, float*, bool vbf16, const GdnShape&, void*) {
  return stub::record("gdn_fwd_h", nullptr, k, hout, vnew, vbf16, false);
}
int launch_gdn_fwd_o(const void* q, const void*, const void*, const float* h, const float*,
                     void* o, float, bool obf16, const GdnShape&, void*) {
  return stub::record("gdn_fwd_o", nullptr, q, h, o, obf16, false);
}
int launch_causal_conv1d(const void* x, const float* weight, const float*, void* out, int64_t,
                         int64_t, int64_t, int, bool bf16_in, bool bf16_out, void*) {
  return stub::record("causal_conv1d", nullptr, x, weight, out, bf16_in, bf16_out);
}

}  // namespace ssd
