// Drives dora_forward and dora_backward (csrc/api.hip, built for the host
// against the stand-in runtime) once each, with the launch named by
// DORA_MOCK_FAIL failing, and checks the stream order the calls left behind:
//   * every launch on the library's side stream is ordered before anything
//     the caller enqueues on its stream after the call returns;
//   * every fork to the side stream is joined back before the call returns.
// Prints one line per call: "<call> rc=<code> launches=<n> ok" or a reason.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <map>
#include <string>

#include "../../include/dora.h"

using mock::Op;

static bool check(const char* what, int rc, hipStream_t caller) {
  const auto& log = mock::log();
  struct Clock { std::map<MockStream*, long> seen; long launches = 0; };
  std::map<MockStream*, Clock> clk;
  std::map<long, std::map<MockStream*, long>> snap;   // record stamp -> recorder's clock
  long n_launch = 0;
  std::vector<size_t> forks;   // positions where a non-caller stream waited on the caller
  std::vector<size_t> joins;   // positions where the caller waited on a non-caller stream
  for (size_t p = 0; p < log.size(); ++p) {
    const Op& o = log[p];
    Clock& c = clk[o.stream];
    if (o.kind == Op::kLaunch) {
      ++c.launches;
      ++n_launch;
    } else if (o.kind == Op::kRecord) {
      auto s = c.seen;
      s[o.stream] = c.launches;
      snap[o.stamp] = s;
    } else {
      for (auto& kv : snap[o.stamp]) c.seen[kv.first] = std::max(c.seen[kv.first], kv.second);
      MockStream* src = o.event->recorded_on;
      if (o.stream != caller && src == caller) forks.push_back(p);
      if (o.stream == caller && src != caller) joins.push_back(p);
    }
  }
  for (auto& kv : clk) {
    if (kv.first == caller) continue;
    const long done = clk[caller].seen[kv.first];
    if (done < kv.second.launches) {
      std::printf("%s rc=%d: caller not ordered after %ld of %ld side-stream launches\n", what, rc,
                  kv.second.launches - done, kv.second.launches);
      return false;
    }
  }
  for (size_t f : forks) {
    bool joined = false;
    for (size_t j : joins) joined |= j > f;
    if (!joined) {
      std::printf("%s rc=%d: fork at log entry %zu never joined\n", what, rc, f);
      return false;
    }
  }
  std::printf("%s rc=%d launches=%ld ok\n", what, rc, n_launch);
  return true;
}

// Whether a launch labelled `label` went to a stream other than the caller's.
static bool launched_beside(const char* label, hipStream_t caller) {
  for (const Op& o : mock::log())
    if (o.kind == Op::kLaunch && o.label == label && o.stream != caller) return true;
  std::printf("%s did not run on the side stream\n", label);
  return false;
}

// Whether every launch labelled `consumer` is ordered after every launch
// labelled `producer` (same stream and later, or reached through recorded
// events); true when either label is absent (a failed call stops early).
static bool ordered_after(const char* consumer, const char* producer) {
  const auto& log = mock::log();
  struct Clock { std::map<MockStream*, long> seen; long launches = 0; };
  struct Launch { MockStream* stream; long index; std::map<MockStream*, long> seen; };
  std::map<MockStream*, Clock> clk;
  std::map<long, std::map<MockStream*, long>> snap;
  std::vector<Launch> prod, cons;
  for (const Op& o : log) {
    Clock& c = clk[o.stream];
    if (o.kind == Op::kLaunch) {
      Launch l{o.stream, c.launches, c.seen};
      if (o.label == producer) prod.push_back(l);
      if (o.label == consumer) cons.push_back(l);
      ++c.launches;
    } else if (o.kind == Op::kRecord) {
      auto s = c.seen;
      s[o.stream] = c.launches;
      snap[o.stamp] = s;
    } else {
      for (auto& kv : snap[o.stamp]) c.seen[kv.first] = std::max(c.seen[kv.first], kv.second);
    }
  }
  for (const Launch& q : cons)
    for (const Launch& p : prod) {
      const bool ok = q.stream == p.stream ? p.index < q.index
                                           : (q.seen.count(p.stream) && q.seen.at(p.stream) > p.index);
      if (!ok) {
        std::printf("%s is not ordered after %s\n", consumer, producer);
        return false;
      }
    }
  return true;
}

int main() {
  MockStream caller_obj{100};
  hipStream_t caller = &caller_obj;
  // large enough that the forward and the backward use the side stream
  dora_shape s{4096, 4096, 64, 4096, DORA_BF16, 2.0f, 0u, 0u};
  char* fake = reinterpret_cast<char*>(uintptr_t(1) << 20);   // never dereferenced
  bool ok = true;

  mock::log().clear();
  int rc = dora_forward(&s, fake, fake, fake, fake, fake, fake, reinterpret_cast<float*>(fake),
                        fake, fake, dora_workspace_bytes(&s, DORA_OP_FORWARD), caller);
  ok &= check("forward", rc, caller);
  ok &= ordered_after("fused_fwd_gemm", "down_proj_xs");
  ok &= ordered_after("fused_fwd_gemm", "cross_gram_proj");
  ok &= ordered_after("cross_gram_proj", "gram_finalize");
  const char* fail = std::getenv("DORA_MOCK_FAIL");
  if (!fail || !*fail) ok &= launched_beside("down_proj_xs", caller);

  mock::log().clear();
  rc = dora_backward(&s, fake, fake, fake, fake, fake, fake, reinterpret_cast<float*>(fake), fake,
                     fake, fake, fake, fake, reinterpret_cast<float*>(fake), fake,
                     dora_workspace_bytes(&s, DORA_OP_BACKWARD), caller);
  ok &= check("backward", rc, caller);
  ok &= ordered_after("t_proj", "bg_scale");
  ok &= ordered_after("dx_gemm", "t_proj");
  ok &= ordered_after("dx_gemm", "compose_bwd");
  ok &= ordered_after("dA_gemm", "t_proj");
  ok &= ordered_after("dm_finalize", "compose_bwd");
  if (!fail || !*fail) ok &= launched_beside("t_proj", caller);
  ok &= ordered_after("dB_gemm", "compose_bwd");
  return ok ? 0 : 1;
}
