// Host-only stand-in for <hip/hip_runtime.h>, for compiling the library's C ABI
// (csrc/api.hip) with g++ in the CPU tests.  Streams and events are plain
// objects; every record and wait is appended to a log that the test replays to
// check stream ordering.  No device code and no HIP runtime are involved.
#pragma once
#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

struct MockStream { int id; };
struct MockEvent { int id; MockStream* recorded_on = nullptr; long stamp = -1; };
typedef MockStream* hipStream_t;
typedef MockEvent* hipEvent_t;
enum hipError_t { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorLaunchFailure = 719 };
constexpr unsigned hipStreamNonBlocking = 1;
constexpr unsigned hipEventDisableTiming = 2;

namespace mock {
struct Op {
  enum Kind { kLaunch, kRecord, kWait } kind;
  MockStream* stream;      // launch / record: the stream; wait: the waiting stream
  MockEvent* event;        // record / wait
  long stamp;              // wait: the stamp of the record it waits for
  std::string label;       // launch
};
std::vector<Op>& log();
MockStream* null_stream();
}  // namespace mock

hipError_t hipGetDevice(int* dev);
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned flags);
hipError_t hipEventCreate(hipEvent_t* e);
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned flags);
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s);
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned flags);
hipError_t hipEventSynchronize(hipEvent_t e);
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b);
