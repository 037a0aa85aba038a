// The stand-in runtime and kernel launchers behind tests/hostmock/hip/hip_runtime.h.
// A launch is a log entry on its stream; DORA_MOCK_FAIL names a launch label
// whose launches fail (nothing is enqueued then, as for a rejected launch).
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <deque>

#include "kernels.h"

namespace mock {
std::vector<Op>& log() {
  static std::vector<Op> v;
  return v;
}
MockStream* null_stream() {
  static MockStream s{0};
  return &s;
}
static std::deque<MockStream>& streams() {
  static std::deque<MockStream> d;
  return d;
}
static std::deque<MockEvent>& events() {
  static std::deque<MockEvent> d;
  return d;
}
static long g_stamp = 0;
}  // namespace mock

using namespace mock;

static MockStream* S(hipStream_t s) { return s ? s : null_stream(); }

hipError_t hipGetDevice(int* dev) { *dev = 0; return hipSuccess; }
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned) {
  streams().push_back(MockStream{(int)streams().size() + 1});
  *s = &streams().back();
  return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t* e) {
  events().push_back(MockEvent{(int)events().size() + 1});
  *e = &events().back();
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) { return hipEventCreate(e); }
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s) {
  e->recorded_on = S(s);
  e->stamp = ++g_stamp;
  log().push_back(Op{Op::kRecord, S(s), e, e->stamp, ""});
  return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned) {
  log().push_back(Op{Op::kWait, S(s), e, e->stamp, ""});
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) { *ms = 0.f; return hipSuccess; }

static hipError_t launch(const char* label, hipStream_t st) {
  const char* f = std::getenv("DORA_MOCK_FAIL");
  if (f && std::strcmp(f, label) == 0) return hipErrorLaunchFailure;
  log().push_back(Op{Op::kLaunch, S(st), nullptr, 0, label});
  return hipSuccess;
}

namespace dora {
GemmPlan plan_gemm(int64_t, int64_t, int64_t, int, bool, bool) { return {2, 2}; }
int64_t gemm_col_slots(int, int64_t N) { return (N + 127) / 128 * 2; }
GemmPlan plan_norm_projection(int64_t, int64_t, int64_t, int64_t) { return {2, 2}; }
int64_t gemm_tile_rows(int, int64_t M) { return (M + 127) / 128; }
size_t gemm_scratch_bytes(int64_t M, int64_t N, int64_t, int, bool, bool) {
  return (size_t)2 * M * N * 4;
}
hipError_t gemm(const GemmProblem&, int, hipStream_t st, const char* label) {
  return launch(label, st);
}
GramPlan gram_bf16_plan(int64_t r, int64_t) { return GramPlan{1, 1, 64, (size_t)(r * r * 4)}; }
hipError_t gram_bf16(const void*, int64_t, int64_t, const GramPlan&, float*, hipStream_t st) {
  return launch("gram_AAt", st);
}
hipError_t gram_bf16_finish(const float*, const GramPlan&, int64_t, float, void*, void*, uint32_t*,
                            int64_t, hipStream_t st) {
  return launch("gram_finalize", st);
}
hipError_t gram_finalize(const float*, int, int64_t, float, int, void*, void*, hipStream_t st,
                         const char* label) {
  return launch(label, st);
}
hipError_t exact_prep(const void*, const float*, const float*, const void*, float, float*, void*,
                      int64_t, int64_t, int, hipStream_t st) {
  return launch("exact_prep", st);
}
hipError_t vera_scale(const void*, const void*, const void*, void*, int64_t, int64_t, int,
                      hipStream_t st) {
  return launch("vera_scale", st);
}
int64_t vera_dd_blocks(int64_t d_out) { return (d_out + 63) / 64; }
hipError_t vera_grads(const void*, const void*, const void*, const void*, void*, void*, float*,
                      int64_t, int64_t, int, hipStream_t st) {
  return launch("vera_grads", st);
}
hipError_t db_combine(const float*, int, const float*, int, const float*, void*, int64_t, int64_t,
                      int, hipStream_t st) {
  return launch("dB_combine", st);
}
hipError_t row_norm(const void*, const void*, const float*, int, float*, int64_t, int64_t, int64_t,
                    int, hipStream_t st) {
  return launch("row_norm", st);
}
hipError_t compose_fwd(void*, const void*, const void*, const float*, int64_t, int64_t, int,
                       hipStream_t st) {
  return launch("compose_fwd", st);
}
hipError_t compose_bwd(const void*, const void*, const void*, const float*, void*, float*, int64_t,
                       int64_t, int64_t, int, hipStream_t st) {
  return launch("compose_bwd", st);
}
hipError_t small_forward(const float*, const float*, const float*, const float*, const float*,
                         float, float*, float*, float*, float*, int64_t, int64_t, int64_t, int64_t,
                         hipStream_t st) {
  const hipError_t e = launch("small_partials", st);
  return e != hipSuccess ? e : launch("small_finish", st);
}
hipError_t scale_b_rows_t(const void*, const void*, const float*, float, void*, int64_t, int64_t,
                          int, hipStream_t st) {
  return launch("bg_scale", st);
}
hipError_t dm_finalize(const float*, int64_t, const void*, float*, int64_t, const DmRecompute&, int,
                       hipStream_t st) {
  return launch("dm_finalize", st);
}
}  // namespace dora
